// Weighted gather + neural compression on bf16 MFMA (gfx950).
//
// For split i: Xhat_i = P X_cat + X_i with X_cat = [X_i; w_1 X_{j_1}; ...; w_k X_{j_k}]
// (papernotes.org Avey-B note, 关键设计 4, eq. 8; retrieved splits scaled by their normalised
// scores per 方法详解/整体框架; residual to the split's own tokens per the paperlayer.ai
// "Avey-B" summary, appendix H). X_cat is never materialised: the K dimension of the GEMM,
// (k+1)S, walks the gathered splits through idx, one 32-token chunk at a time, the retrieved
// blocks 1..k first and the split's own block 0 last. The weights are applied to the fp32
// accumulator between blocks: after block r it is multiplied by w_r / w_{r+1}, after block k
// by w_k, so that it ends as sum_r w_r (P_r X_r) + P_0 X_0. This holds whenever every weight is
// a positive normal number in [2^-60, 2^60] (top-k weights are, unless a score is zero or
// negative); otherwise each P fragment of block r is multiplied by w_r as it is read (rounded
// to bf16), using (w P_r) X = P_r (w X).
//
// The product is computed transposed, C[f][s] = sum_kk X_cat[kk][f] P[s][kk], so that each lane
// of the result owns one output token and four consecutive features (8-byte stores). Both
// operands stream global -> LDS by direct copies through a 4-stage ring (three chunks in flight
// while one is multiplied): gathered X rows token-major, P rows K-contiguous. X^T fragments
// are read with the LDS transpose read (ds_read_b64_tr_b16): within each group of 16 lanes,
// lane i receives element (i & 3) of the 8-byte rows addressed by lanes (i >> 2) + 4k, k = 0..3,
// so pointing lane j at token (j >> 2), features 4 (j & 3) .. + 3 hands lane i four consecutive
// tokens of feature i.
//
// Workgroup: 256 threads = 4 waves in a 2 x 2 grid over a 256-feature x 128-token output tile,
// each wave 128 features x 64 tokens (8 MFMA 32x32x16 blocks), with a 3-stage ring of 24 KiB
// stages, so that two workgroups share a CU: one's epilogue (residual loads and stores) then
// overlaps the other's MFMAs.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

constexpr int TF = 256;   // features per tile
constexpr int TS = 128;   // output tokens per tile
constexpr int KH = 32;    // tokens of X_cat (K) per chunk
constexpr int XB = TF * 2;            // bytes per X row in LDS (one token of the feature tile)
constexpr int XS = KH * XB;           // X part of a stage (16 KiB)
constexpr int PB = KH * 2;            // bytes per P row in LDS (one chunk of one output token)
constexpr int STAGE = XS + TS * PB;   // 24 KiB

// X rows: the 32-byte piece c of LDS row t sits at c ^ (2 (t & 3)). A transpose read covers 4
// consecutive rows x two adjacent pieces per 32 lanes: 8 distinct 32-byte slots of a 256-byte
// bank window. P rows: as the MaxSim operands, 16-byte piece c of row r at c ^ ((r >> 2) & 3).
__device__ __forceinline__ uint32_t sw4(int r) { return (uint32_t)((r >> 2) & 3); }

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* base, uint32_t off) {
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

// Eight bf16 values times w, rounded to bf16 (round to nearest even).
__device__ __forceinline__ uint4 scale8(uint4 v, float w) {
  uint4 o;
  o.x = pack_bf16(bf16lo(v.x) * w, bf16hi(v.x) * w);
  o.y = pack_bf16(bf16lo(v.y) * w, bf16hi(v.y) * w);
  o.z = pack_bf16(bf16lo(v.z) * w, bf16hi(v.z) * w);
  o.w = pack_bf16(bf16lo(v.w) * w, bf16hi(v.w) * w);
  return o;
}

struct CompressParams {
  const uint16_t* x;
  const int32_t* idx;
  const float* w;
  const uint16_t* P;
  uint16_t* xhat;
  int64_t N, ld_x, ld_out, tiles;
  int d, S, k, n_s, s_tiles, f_tiles, residual;
  LayerEpi epi;
};

// This wave's copies except the newest n are complete, then a workgroup barrier.
#define WAIT_KEEP(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

constexpr int MAXBLK = kCompressMaxBlocks;   // k + 1 <= MAXBLK (checked by the caller)
constexpr int kEmptyBlock = -(1 << 30);      // first token of an empty block: every copy is out of range

__global__ void __launch_bounds__(256, 2) compress_bf16_kernel(CompressParams a) {
  __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE];
  __shared__ int s_tok0[MAXBLK];     // first token of block r's source split
  __shared__ float s_wt[MAXBLK];     // weight applied to block r's P fragments
  __shared__ float s_ps[MAXBLK];     // accumulator factor after block r's last chunk
  __shared__ int s_slow;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 1, wn = wave & 1;

  const int64_t L = xcd_remap(blockIdx.x, a.tiles);
  const int ft = (int)(L % a.f_tiles);
  const int64_t rest = L / a.f_tiles;
  const int stl = (int)(rest % a.s_tiles);
  const int64_t split = rest / a.s_tiles;
  const int64_t b = split / a.n_s;
  const int i = (int)(split % a.n_s);

  const uint16_t* xb = a.x + b * a.N * a.ld_x;
  const __amdgpu_buffer_rsrc_t xr = make_rsrc(xb, (uint32_t)(a.N * a.ld_x * 2));
  const int KP = (a.k + 1) * a.S;          // row length of P
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P, (uint32_t)((int64_t)a.S * KP * 2));
  const int32_t* idx_i = a.idx + split * a.k;
  const float* w_i = a.w + split * a.k;
  const int nk = KP / KH;
  const int nk3 = (nk + 2) / 3 * 3;
  const int f_base = ft * TF;

  // Source split and weights of every block, staged in LDS before any copy is issued: inside
  // the K loop only the copies may count as vector-memory operations, so that the copy waits
  // count exactly 4 per chunk.
  if (tid == 0) s_slow = 0;
  __syncthreads();
  for (int r = tid; r <= a.k; r += 256) {
    const int src = r ? idx_i[r - 1] : i;
    // a negative index is an empty block (zero rows, as the unidirectional ranker pads its
    // selection): its copies load zeros and its weight is taken as 1, which changes nothing
    s_tok0[r] = src < 0 ? kEmptyBlock : min(src, a.n_s - 1) * a.S;
    const float wr = (r && src >= 0) ? w_i[r - 1] : 1.f;
    s_wt[r] = wr;
    if (!(wr >= 0x1p-60f && wr <= 0x1p60f)) s_slow = 1;   // also catches NaN
  }
  __syncthreads();
  const bool slow = s_slow != 0;
  for (int r = tid; r <= a.k; r += 256) {
    const float wr = s_wt[r];
    float ps = 1.f;
    if (!slow && r >= 1) ps = r < a.k ? wr / s_wt[r + 1] : wr;
    s_ps[r] = ps;
    if (!slow) s_wt[r] = 1.f;
  }
  __syncthreads();
  // Chunk c of the K loop covers block (c / cpb + 1) mod (k + 1): blocks 1..k, then block 0.
  const int cpb = a.S / KH;
  auto chunk_block = [&](int c, int& r, int& kk0) {
    const int q = c / cpb;
    r = q < a.k ? q + 1 : 0;
    kk0 = r * a.S + (c - q * cpb) * KH;
  };
  // Source tokens and fragment weight of chunk c.
  auto chunk_src = [&](int c, int& tok0, float& wt) {
    int r, kk0;
    chunk_block(c, r, kk0);
    tok0 = s_tok0[r] + (kk0 - r * a.S);
    wt = s_wt[r];
  };

  // Chunk kc into stage st, 6 copies per wave: X tokens 8w .. 8w + 7 (n = 0..3, 2 tokens per
  // copy, 1 KiB) and P rows 32w .. 32w + 31 (n = 4, 5, 16 rows per copy). Lane terms are
  // recomputed per chunk (laundered so they are not hoisted into long-lived registers). Tokens
  // past N, features past d and rows past S load zeros.
  auto copy_chunk = [&](int kc, uint8_t* st, bool valid, int n) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    if (n < 4) {
      int tok0 = 0;
      float wt_unused;
      chunk_src(kc, tok0, wt_unused);
      const int t = wave * 8 + n * 2 + (ln >> 5);                  // row in the stage
      const int p = ln & 31;                                       // 16-byte position in the row
      const int c = (p >> 1) ^ (2 * (t & 3));                      // logical 32-byte piece
      const int f = f_base + c * 16 + (p & 1) * 8;
      const int64_t tok = (int64_t)tok0 + t;
      const bool ok = valid && tok >= 0 && tok < a.N && f < a.d;
      dma16(xr, st + (wave * 8 + n * 2) * XB, ok ? (uint32_t)((tok * a.ld_x + f) * 2) : OOB, 0);
    } else {
      const int r0 = wave * 32 + (n - 4) * 16;
      const int sub = ln >> 2;
      const int row = r0 + sub;                                    // output token in the tile
      const int s = stl * TS + row;
      const uint32_t piece = (uint32_t)((ln & 3) ^ (int)sw4(row));
      const bool ok = valid && s < a.S;
      int r, kk0;
      chunk_block(kc, r, kk0);
      dma16(pr, st + XS + r0 * PB, ok ? (uint32_t)s * (uint32_t)KP * 2u + 16u * piece : OOB,
            (uint32_t)kk0 * 2u);
    }
  };

  // Fragment offsets. A (X^T): lane l of a transpose read points at token
  // 8 (l >> 5) + ((l & 15) >> 2) (+ 16 ks + 4 q), features 4 (l & 3) of piece
  // wm * 8 + 2 mb + ((l >> 4) & 1), swizzled by the token's low bits.
  uint32_t offA[4];
  {
    const int s2 = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    const uint32_t row = (uint32_t)(8 * (lane >> 5) + ((lane & 15) >> 2)) * XB;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      offA[mb] = row + (uint32_t)((wm * 8 + 2 * (mb ^ s2) + g1) << 5) + 8u * (lane & 3);
  }
  uint32_t offB[2];
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int rb = wn * 64 + (lane & 31);
    offB[ks] = (uint32_t)XS + (uint32_t)rb * PB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(rb)) << 4);
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mb][nb][v] = 0.f;

  // One chunk of MFMAs from stage st (weight wt of its block), with the 6 copies of chunk nkc
  // into stage dst spread between its MFMA groups.
  auto compute_copy = [&](const uint8_t* st, float wt, int nkc, uint8_t* dst, bool valid) {
    uint4 ra[2][4], rb[2][2];
    auto fetch = [&](int ks) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        const uint2 lo = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks) * XB);
        const uint2 hi = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks + 4) * XB);
        ra[ks][mb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const uint4 v = lds_read16(st, offB[ks] + nb * 32 * PB);
        rb[ks][nb] = wt == 1.f ? v : scale8(v, wt);
      }
    };
    fetch(0);
    copy_chunk(nkc, dst, valid, 4);
    copy_chunk(nkc, dst, valid, 5);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int mb = 2 * h; mb < 2 * h + 2; ++mb)
#pragma unroll
          for (int nb = 0; nb < 2; ++nb)
            acc[mb][nb] = mfma32(as_bf16x8(ra[ks][mb]), as_bf16x8(rb[ks][nb]), acc[mb][nb]);
        if (ks == 0 && h == 0) fetch(1);
        copy_chunk(nkc, dst, valid, 2 * ks + h);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  auto weight = [&](int kc) {
    int t0;
    float wt = 1.f;
    if (kc < nk) chunk_src(kc, t0, wt);
    return wt;
  };
  // After chunk c: at the last chunk of a block, multiply the accumulator by the block's factor.
  auto post = [&](int c) {
    if (c >= nk || (c + 1) % cpb) return;
    int r, kk0;
    chunk_block(c, r, kk0);
    const float f = s_ps[r];
    if (f == 1.f) return;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] *= f;
  };

  for (int n = 0; n < 6; ++n) copy_chunk(0, st0, true, n);
  for (int n = 0; n < 6; ++n) copy_chunk(1, st1, 1 < nk, n);
  // Every chunk is exactly 6 copies per wave: WAIT_KEEP(6) leaves the next chunk in flight.
  for (int kc = 0; kc < nk3; kc += 3) {
    WAIT_KEEP(6);
    compute_copy(st0, weight(kc), kc + 2, st2, kc + 2 < nk);
    post(kc);
    WAIT_KEEP(6);
    compute_copy(st1, weight(kc + 1), kc + 3, st0, kc + 3 < nk);
    post(kc + 1);
    WAIT_KEEP(6);
    compute_copy(st2, weight(kc + 2), kc + 4, st1, kc + 4 < nk);
    post(kc + 2);
  }
  wait_vmem();   // the zero-filled copies issued past the last chunk land before the exit

  // Epilogue: lane owns token s, four consecutive features per (mb, g). The residual rows of a
  // token block are all loaded before any store (stores could alias them as far as the
  // compiler knows, which would otherwise serialise one load round trip per store). Without
  // the residual the loads are out of range and return zeros without touching memory. The
  // layer epilogue (bias per token position, activation) is applied last.
  uint16_t* ob = a.xhat + b * a.N * a.ld_out;
  const bool relu = a.epi.act != 0;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int s = stl * TS + wn * 64 + nb * 32 + (lane & 31);
    const int64_t tok = (int64_t)i * a.S + s;
    const bool tok_ok = s < a.S && tok < a.N;
    const bool res_ok = tok_ok && a.residual;
    const float bv = (tok_ok && a.epi.bias) ? a.epi.bias[s] : 0.f;
    uint2 res[4][4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f_base + wm * 128 + mb * 32 + g * 8 + (lane >> 5) * 4;
        res[mb][g] = buf_load8(xr, (res_ok && f < a.d) ? (uint32_t)((tok * a.ld_x + f) * 2) : OOB, 0);
      }
    auto out = [&](float acc, float r) {
      const float v = (acc + r) + bv;
      return relu ? fmaxf(v, 0.f) : v;
    };
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int f = f_base + wm * 128 + mb * 32 + g * 8 + (lane >> 5) * 4;
        const uint2 r = res[mb][g];
        const float v0 = out(acc[mb][nb][g * 4 + 0], bf16lo(r.x));
        const float v1 = out(acc[mb][nb][g * 4 + 1], bf16hi(r.x));
        const float v2 = out(acc[mb][nb][g * 4 + 2], bf16lo(r.y));
        const float v3 = out(acc[mb][nb][g * 4 + 3], bf16hi(r.y));
        if (tok_ok && f < a.d)
          *reinterpret_cast<uint2*>(ob + tok * a.ld_out + f) = make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
      }
  }
}

}  // namespace

hipError_t launch_compress_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld_x, int S, int k,
                                const int32_t* idx, const float* w, const uint16_t* P, int residual, uint16_t* xhat,
                                int64_t ld_out, hipStream_t stream, LayerEpi epi) {
  CompressParams p;
  p.x = x; p.idx = idx; p.w = w; p.P = P; p.xhat = xhat;
  p.N = N; p.ld_x = ld_x; p.ld_out = ld_out;
  p.d = d; p.S = S; p.k = k;
  p.n_s = (int)((N + S - 1) / S);
  p.s_tiles = (S + TS - 1) / TS;
  p.f_tiles = (d + TF - 1) / TF;
  p.residual = residual;
  p.epi = epi;
  p.tiles = B * p.n_s * p.s_tiles * p.f_tiles;
  hipLaunchKernelGGL(compress_bf16_kernel, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
