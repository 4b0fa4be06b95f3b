// Weighted gather + neural compression on bf16 MFMA (gfx950).
//
// For split i: Xhat_i = P X_cat + X_i with X_cat = [X_i; w_1 X_{j_1}; ...; w_k X_{j_k}]
// (papernotes.org Avey-B note, 关键设计 4, eq. 8; retrieved splits scaled by their normalised
// scores per 方法详解/整体框架; residual to the split's own tokens per the paperlayer.ai
// "Avey-B" summary, appendix H). X_cat is never materialised: the K dimension of the GEMM,
// (k+1)S, walks the gathered splits through idx, one 32-token chunk at a time, the retrieved
// blocks first and the split's own block last. The weights are applied to the fp32 accumulator
// between blocks: with the retrieved blocks taken in ascending order of |w| as w_1..w_k, after
// block r it is multiplied by w_r / w_{r+1}, after block k by w_k, so that it ends as
// sum_r w_r (P_r X_r) + P_0 X_0 (P_r: the columns of P for the block's rank in the selection).
// Every factor lies in [-1, 1] except the last, which cannot overflow a finite result; a factor
// that underflows to zero drops a block whose term is below 2^-149 of a later one. Blocks that
// add nothing (an empty block, a zero weight) come after the others with factor 1; a NaN or
// infinite weight comes last and makes the split's outputs non-finite, as it makes w X.
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
// Two kernels share this scheme: a persistent one (namespace unit, below) for problems with at
// least one 256-feature x 256-token unit per CU, and the tiled one described here for smaller
// problems, where its smaller tiles keep more CUs busy.
//
// Tiled kernel: 256 threads = 4 waves in a 2 x 2 grid over a 256-feature x 128-token output tile,
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

// Order of a retrieved block (index src, weight w) in the K loop: ascending |w| (the bits of a
// finite |w| order as the values do), then the blocks that contribute nothing (an empty block,
// negative index; a zero weight), then those with a non-finite weight.
constexpr uint32_t kKeyNone = 0x7F800000u;
__device__ __forceinline__ uint32_t block_key(int src, float w) {
  if (src < 0 || w == 0.f) return kKeyNone;
  const uint32_t m = __float_as_uint(w) & 0x7FFFFFFFu;
  return m < kKeyNone ? m : kKeyNone + 1u;
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
  __shared__ int s_col0[MAXBLK];     // first column of P that multiplies block r
  __shared__ float s_wt[MAXBLK];     // weight of block r
  __shared__ float s_ps[MAXBLK];     // accumulator factor after block r's last chunk

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
  // chunks per block: the last one of a block is partial when S % 32 != 0 (its rows past S load
  // zeros, so the columns of P they meet, the next block's, add nothing)
  const int cpb = (a.S + KH - 1) / KH;
  const int nk = (a.k + 1) * cpb;
  const int nk3 = (nk + 2) / 3 * 3;
  const int f_base = ft * TF;

  // Block table, staged in LDS before any copy is issued: inside the K loop only the copies may
  // count as vector-memory operations, so that the copy waits count whole chunks. Slot 0
  // is the split's own block; the retrieved blocks follow in block_key order, so that every
  // accumulator factor w_r / w_(r+1) lies in [-1, 1]. The sort keys sit in s_ps until the
  // factors replace them.
  uint32_t* s_key = reinterpret_cast<uint32_t*>(s_ps);
  for (int r = tid + 1; r <= a.k; r += 256) s_key[r] = block_key(idx_i[r - 1], w_i[r - 1]);
  __syncthreads();
  for (int r = tid; r <= a.k; r += 256) {
    if (r == 0) {
      s_tok0[0] = i * a.S;
      s_col0[0] = 0;
      s_wt[0] = 1.f;
      continue;
    }
    const uint32_t key = s_key[r];
    int pos = 1;   // 1 + the number of retrieved blocks ordered before this one
    for (int j = 1; j <= a.k; ++j) pos += (s_key[j] < key || (s_key[j] == key && j < r)) ? 1 : 0;
    const bool none = key == kKeyNone;
    // an empty block (zero rows, as the unidirectional ranker pads its selection) or a zero
    // weight: its copies load zeros and its factor is 1
    s_tok0[pos] = none ? kEmptyBlock : min(idx_i[r - 1], a.n_s - 1) * a.S;
    s_col0[pos] = r * a.S;   // P keeps the rank order of the selection
    s_wt[pos] = none ? 1.f : w_i[r - 1];
  }
  __syncthreads();
  for (int r = tid; r <= a.k; r += 256) s_ps[r] = r == 0 ? 1.f : r < a.k ? s_wt[r] / s_wt[r + 1] : s_wt[r];
  __syncthreads();
  // Chunk c of the K loop covers slot (c / cpb + 1) mod (k + 1): slots 1..k, then slot 0; j is
  // its offset within the block.
  auto chunk_block = [&](int c, int& r, int& j) {
    const int q = c / cpb;
    r = q < a.k ? q + 1 : 0;
    j = (c - q * cpb) * KH;
  };

  // Chunk kc into stage st, 6 copies per wave: X tokens 8w .. 8w + 7 (n = 0..3, 2 tokens per
  // copy, 1 KiB) and P rows 32w .. 32w + 31 (n = 4, 5, 16 rows per copy). Lane terms are
  // recomputed per chunk (laundered so they are not hoisted into long-lived registers). Tokens
  // past N or past their block's S tokens, features past d and rows past S load zeros.
  auto copy_chunk = [&](int kc, uint8_t* st, bool valid, int n) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    int r, j;
    chunk_block(kc, r, j);
    if (n < 4) {
      const int tok0 = s_tok0[r] + j;
      const int t = wave * 8 + n * 2 + (ln >> 5);                  // row in the stage
      const int p = ln & 31;                                       // 16-byte position in the row
      const int c = (p >> 1) ^ (2 * (t & 3));                      // logical 32-byte piece
      const int f = f_base + c * 16 + (p & 1) * 8;
      const int64_t tok = (int64_t)tok0 + t;
      const bool ok = valid && tok >= 0 && tok < a.N && j + t < a.S && f < a.d;
      dma16(xr, st + (wave * 8 + n * 2) * XB, ok ? (uint32_t)((tok * a.ld_x + f) * 2) : OOB, 0);
    } else {
      const int r0 = wave * 32 + (n - 4) * 16;
      const int sub = ln >> 2;
      const int row = r0 + sub;                                    // output token in the tile
      const int s = stl * TS + row;
      const uint32_t piece = (uint32_t)((ln & 3) ^ (int)sw4(row));
      const bool ok = valid && s < a.S;
      dma16(pr, st + XS + r0 * PB, ok ? (uint32_t)s * (uint32_t)KP * 2u + 16u * piece : OOB,
            (uint32_t)(s_col0[r] + j) * 2u);
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

  // One chunk of MFMAs from stage st, with the 6 copies of chunk nkc into stage dst spread
  // between its MFMA groups.
  auto compute_copy = [&](const uint8_t* st, int nkc, uint8_t* dst, bool valid) {
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
        rb[ks][nb] = lds_read16(st, offB[ks] + nb * 32 * PB);
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
  // After chunk c: at the last chunk of a block, multiply the accumulator by the block's factor.
  auto post = [&](int c) {
    if (c >= nk || (c + 1) % cpb) return;
    int r, j;
    chunk_block(c, r, j);
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
    compute_copy(st0, kc + 2, st2, kc + 2 < nk);
    post(kc);
    WAIT_KEEP(6);
    compute_copy(st1, kc + 3, st0, kc + 3 < nk);
    post(kc + 1);
    WAIT_KEEP(6);
    compute_copy(st2, kc + 4, st1, kc + 4 < nk);
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

// ---------------------------------------------------------------------------------------------
// Persistent variant for problems with at least one unit per CU. A unit is 256 features x all
// output tokens of a split (256 of them; at S = 512 two units per split), one 8-wave workgroup
// per CU in a 2 x 4 wave grid (each wave 128 features x 64 tokens, as above), a 4-stage ring of
// 32 KiB (three chunks in flight) and the next unit's first three chunks copied while the
// current one finishes. Compared with the tiled kernel, each gathered X row is staged once per
// feature tile instead of once per 128 output tokens.
//   * Features of wave (wm, mb): 128 wm + 32 mb + (0..31), so that each wave holds two whole
//     64-feature slices (128-byte row pieces) of its 64 tokens.
//   * Residual: the split's own block comes last; in the chunk of it that holds a wave's token
//     block nb, 8 more MFMAs of that chunk's X^T fragments with an identity B operand add
//     X_i[s][f] to C[f][s] exactly.
//   * Epilogue, through stage 3, each wave through its own 4 KiB of it (one barrier per unit), in
//     four rounds of 32 tokens x 64 features: lanes write their 4-feature groups into a bf16
//     tile, then 8 lanes per token store whole 128-byte row pieces (scattered 8-byte stores
//     would cost a write request per lane, and 64-byte pieces measured slower).
//   * Source splits and weights of the next unit are read with scalar loads into a second LDS
//     table, so that the copies stay the only vector-memory operations of the K loop. When the
//     copies move on to a unit, its block table is loaded once into one VGPR (lane r: block r's
//     first token); each chunk then takes its token base with a lane read, with no LDS load
//     (whose wait would also drain the fragment reads in flight).
//   * The per-chunk bookkeeping is kept to scalar integer work without divisions (chunk ->
//     block by a multiply-shift) and the copy offsets to 32-bit arithmetic without branches.
namespace unit {

constexpr int TU = 256;                 // output tokens per unit
constexpr int kMaxBlocks = 64;          // k + 1: one lane of a VGPR per block of the unit's table
constexpr int USTAGE = XS + TU * PB;    // 32 KiB: 32 X rows of 256 features + 256 P rows

struct UnitPos {
  int64_t b;
  int i, su, f_base;
};

typedef const __attribute__((address_space(4))) int32_t* sc_i32;
typedef const __attribute__((address_space(4))) float* sc_f32;

// Compile-time pipeline position 0..3 of a chunk (its stage).
template <int P>
using Pos = std::integral_constant<int, P>;

// CPB: chunks per block (S / 32) as a compile-time constant, or 0 for any S; kRelu: the layer
// epilogue's activation.
template <int CPB, bool kRelu>
__global__ void __launch_bounds__(512, 1) compress_unit_kernel(CompressParams a) {
  __shared__ __align__(16) uint8_t st0[USTAGE], st1[USTAGE], st2[USTAGE], st3[USTAGE];
  __shared__ int s_tok0[2][MAXBLK];   // per unit (two tables): first token of block r's split
  __shared__ float s_wt[2][MAXBLK];   // weight of block r
  __shared__ int s_col0[2][MAXBLK];   // first column of P that multiplies block r
  __shared__ float s_bias[512];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6), wm = wave >> 2, wn = wave & 3;

  // XCD x owns units [xs, xs + cnt); its workgroup l takes every Gx-th of them from l.
  const int G = gridDim.x, wg = blockIdx.x, xcd = wg % NXCD, l = wg / NXCD;
  const int Gx = (G - xcd + NXCD - 1) / NXCD;
  const int64_t q8 = a.tiles / NXCD, r8 = a.tiles % NXCD;
  const int64_t xs = xcd * q8 + (xcd < r8 ? xcd : r8), cnt = q8 + (xcd < r8 ? 1 : 0);
  int64_t t = l;
  if (t >= cnt) return;

  const int KP = (a.k + 1) * a.S;
  // chunks per block, even (the residual's pipeline parity below relies on it): when S is not a
  // multiple of 64 the last chunks of a block are partial or empty, their rows past S zeros
  const int cpb = CPB ? CPB : (a.S + 2 * KH - 1) / (2 * KH) * 2;
  const int nk = (a.k + 1) * cpb;
  const int nk4 = (nk + 3) / 4 * 4;       // padded with zero chunks: every unit starts on stage 0
  // floor(c / cpb) as (c * cpb_magic) >> 20: exact while c * (cpb_magic * cpb - 2^20) < 2^20,
  // i.e. for c < 2^16 with cpb <= 16, far above any chunk index here
  const uint32_t cpb_magic = ((1u << 20) + (uint32_t)cpb - 1u) / (uint32_t)cpb;
  const __amdgpu_buffer_rsrc_t pr = make_rsrc(a.P, (uint32_t)((int64_t)a.S * KP * 2));

  auto unit_pos = [&](int64_t tl) {
    UnitPos u;
    const int64_t L = xs + tl;
    const int ft = (int)(L % a.f_tiles);
    const int64_t rest = L / a.f_tiles;
    u.su = (int)(rest % a.s_tiles);
    const int64_t split = rest / a.s_tiles;
    u.b = split / a.n_s;
    u.i = (int)(split % a.n_s);
    u.f_base = ft * TF;
    return u;
  };
  // Block table of a unit: slot 0 is the split's own block (weight 1), the retrieved blocks
  // follow in block_key order, so that every factor w_r / w_(r+1) the accumulator is multiplied
  // by lies in [-1, 1].
  auto fill_table = [&](const UnitPos& u, int bf) {
    const int64_t row = (u.b * a.n_s + u.i) * (int64_t)a.k;
    for (int r = wave; r <= a.k; r += 8) {
      if (r == 0) {
        s_tok0[bf][0] = u.i * a.S;
        s_wt[bf][0] = 1.f;
        s_col0[bf][0] = 0;
        continue;
      }
      const int src = ((sc_i32)a.idx)[row + r - 1];
      const float wr = ((sc_f32)a.w)[row + r - 1];
      const uint32_t key = block_key(src, wr);
      int pos = 1;   // 1 + the number of retrieved blocks ordered before this one
      for (int j = 1; j <= a.k; ++j) {
        const uint32_t kj = block_key(((sc_i32)a.idx)[row + j - 1], ((sc_f32)a.w)[row + j - 1]);
        pos += (kj < key || (kj == key && j < r)) ? 1 : 0;
      }
      const bool none = key == kKeyNone;
      s_tok0[bf][pos] = none ? kEmptyBlock : min(src, a.n_s - 1) * a.S;
      s_wt[bf][pos] = none ? 1.f : wr;
      s_col0[bf][pos] = r * a.S;   // P keeps the rank order of the selection
    }
  };
  s_bias[tid] = (a.epi.bias && tid < a.S) ? a.epi.bias[tid] : 0.f;

  // ---- copy side: the unit whose chunks are being copied (the next one near a unit's end)
  __amdgpu_buffer_rsrc_t xr;
  int c_su = 0, c_fb = 0;
  // lane r: first token of block r of the copy unit, and its first column of P (the launcher
  // ensures k + 1 <= 64)
  int vtok = 0, vcol = 0;
  // Each lane's copy offsets for the copy unit, less the chunk's terms (which go in the copies'
  // scalar offsets), with bit 31 set where the lane is out of range whatever the chunk: X row
  // 4 w + 2 n + (lane >> 5) at the lane's feature (n = 0, 1), P row 32 w + 16 (n - 2) +
  // (lane >> 2) (n = 2, 3). A copy then costs at most a compare and a select.
  uint32_t c_off[4] = {0u, 0u, 0u, 0u};
  auto set_copy_unit = [&](const UnitPos& u, int bf) {
    xr = make_rsrc(a.x + u.b * a.N * a.ld_x, (uint32_t)(a.N * a.ld_x * 2));
    c_su = u.su;
    c_fb = u.f_base;
    vtok = lane <= a.k ? s_tok0[bf][lane] : 0;
    vcol = lane <= a.k ? s_col0[bf][lane] : 0;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int tr = wave * 4 + n * 2 + (lane >> 5);
      const int p = lane & 31;
      const int fl = ((p >> 1) ^ (2 * (tr & 3))) * 16 + (p & 1) * 8;
      c_off[n] = ((uint32_t)tr * (uint32_t)a.ld_x + (uint32_t)(c_fb + fl)) * 2u | ((uint32_t)!(fl < a.d - c_fb) << 31);
    }
#pragma unroll
    for (int n = 2; n < 4; ++n) {
      const int row = wave * 32 + (n - 2) * 16 + (lane >> 2);
      const int s = c_su * TU + row;
      const uint32_t piece = (uint32_t)((lane & 3) ^ (int)sw4(row));
      c_off[n] = ((uint32_t)s * (uint32_t)KP * 2u + 16u * piece) | ((uint32_t)!(s < a.S) << 31);
    }
  };
  // Chunk c covers block (c / cpb + 1) mod (k + 1): blocks 1..k, then block 0.
  auto chunk_block = [&](int c, int& r, int& j) {
    const int q = CPB ? c / CPB : (int)(((uint32_t)c * cpb_magic) >> 20);
    r = q < a.k ? q + 1 : 0;
    j = c - q * cpb;
  };
  // First token (x), first column of P (y) and the block's rows left from the chunk's first (z)
  // of chunk kc: lane reads instead of LDS loads, whose wait would also drain the fragment reads.
  auto chunk_src = [&](int kc) {
    int r, j;
    chunk_block(kc, r, j);
    return make_int3(__builtin_amdgcn_readlane(vtok, r) + j * KH, __builtin_amdgcn_readlane(vcol, r) + j * KH,
                     a.S - j * KH);
  };
  // Copy n of chunk kc into stage st: n = 0, 1 are X rows 4 w + 2 n, + 1 (1 KiB), n = 2, 3 are
  // P rows 32 w + 16 (n - 2) .. + 15. Tokens past N or past their block's S tokens, features past
  // d and rows past S load zeros:
  // their offset gets the high bit, past the descriptor's range (a sequence and P are < 2^31
  // bytes), so that the offsets are plain 32-bit arithmetic without a branch.
  // The chunk's terms go in the scalar offset, zero for a chunk out of range, so that bit 31 of a
  // lane's offset alone keeps it out of range (the sums stay below 2^32: every offset inside a
  // sequence or P is below 2^31).
  auto copy = [&](uint8_t* st, bool valid, int n, int3 src) {
    if (n < 2) {
      // X rows src.x + 4 w + 2 n + (lane >> 5): in range while below N and below the block's
      // src.z rows; an empty block's first token is negative and takes the whole chunk out
      const int n_tok = (int)a.N;   // below 2^30 (host checks): 32-bit compares stay scalar
      const bool cok = valid && src.x >= 0 && src.x < n_tok;
      const int bound = cok ? min(src.z, n_tok - src.x) - (wave * 4 + n * 2) : 0;
      int lh = lane >> 5;
      asm volatile("" : "+v"(lh));
      const uint32_t vo = lh < bound ? c_off[n] : OOB;
      dma16(xr, st + (wave * 4 + n * 2) * XB, vo, cok ? (uint32_t)src.x * (uint32_t)a.ld_x * 2u : 0u);
    } else {
      const int r0 = wave * 32 + (n - 2) * 16;
      dma16(pr, st + XS + r0 * PB, c_off[n] | (valid ? 0u : OOB), valid ? (uint32_t)src.y * 2u : 0u);
    }
  };
  auto dma = [&](int kc, uint8_t* st, bool valid) {
    const int3 src = chunk_src(kc);
#pragma unroll
    for (int n = 0; n < 4; ++n) copy(st, valid, n, src);
  };

  // ---- fragments (transpose reads of X for A, P rows for B), feature blocks 128 wm + 32 mb
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
  int bf = 0, cur_su = 0;
  int rc0 = -1, rc1 = -1;   // the chunks of the current unit that add the residual (token blocks 0, 1)
  f32x16 acc[4][2];
  uint4 ra0[4], rb0[2], ra1[4], rb1[2];
  auto fetchA = [&](const uint8_t* st, int ks, uint4 (&ra)[4]) {
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const uint2 lo = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks) * XB);
      const uint2 hi = lds_read_tr8(st, offA[mb] + (uint32_t)(16 * ks + 4) * XB);
      ra[mb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  auto fetchB = [&](const uint8_t* st, int ks, uint4 (&rb)[2]) {
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) rb[nb] = lds_read16(st, offB[ks] + nb * 32 * PB);
  };

  // ---- compute side: the unit being multiplied
  // After chunk c: at the last chunk of a retrieved block r, multiply the accumulator by
  // w_r / w_{r+1} (by w_k after block k).
  auto post = [&](int c) {
    if (c >= nk) return;
    int r, j;
    chunk_block(c, r, j);
    if (j != cpb - 1 || r == 0) return;
    const float f = r < a.k ? s_wt[bf][r] / s_wt[bf][r + 1] : s_wt[bf][r];
    if (f == 1.f) return;
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] *= f;
  };
  // Residual. Identity fragment of k-step ks: lane l (column l & 31) holds 1.0 at element
  // (l & 31) - 16 ks - 8 (l >> 5) when that lies in 0..7. Token block nb of this wave sits in
  // chunk k cpb + 8 su + 2 wn + nb; block 0 starts on an even chunk (cpb is even), so that chunk
  // is at an odd pipeline position exactly when nb = 1.
  // The fragment is built where it is used (from a laundered lane index), so that it does not
  // hold 8 registers across the K loop.
  auto id_frag = [&](int ks) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int j = (ln & 31) - 16 * ks - 8 * (ln >> 5);
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) wv[q] = (j >> 1) == q ? ((j & 1) ? 0x3F800000u : 0x00003F80u) : 0u;
    return make_uint4(wv[0], wv[1], wv[2], wv[3]);
  };
  auto res_chunk = [&](int nb) {
    const int jt = cur_su * 8 + 2 * wn + nb;
    return jt < cpb ? a.k * cpb + jt : -1;
  };
  auto res_mfma = [&](auto POS, bool on, const uint4 (&ra)[4], int ks) {
    if (on) {
      const uint4 id = id_frag(ks);
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
        acc[mb][POS.value & 1] = mfma32(as_bf16x8(ra[mb]), as_bf16x8(id), acc[mb][POS.value & 1]);
    }
  };

  // One chunk c from stage st at position POS (k-step-0 fragments already in ra0 / rb0). The 4
  // copies of chunk kc of the copy unit into dst go between the MFMA groups; with next, the
  // next chunk's wait and barrier come before the last group and its first fragments are read
  // under it.
  const f32x16 zero16 = {};
  // FIRST: the unit's first chunk, whose k-step-0 MFMAs start the accumulators from zero (an
  // inline constant) instead of reading them, so that nothing has to clear them.
  // late: the previous unit's 16 epilogue stores were issued after the copies of the chunk that
  // `next` waits for, and may stay in flight as well.
  // next is nullptr for the unit's last chunk; its type decides at compile time (a run-time test
  // of the stage pointer, which the compiler cannot prove non-null, put a branch into every chunk).
  auto compute_pipe = [&](auto FIRST, auto POS, const uint8_t* st, int c, int kc, uint8_t* dst, bool valid,
                          auto next, bool late) {
    constexpr bool kHasNext = !std::is_same_v<decltype(next), std::nullptr_t>;
    const int3 src = chunk_src(kc);
    const bool ron = (c == rc0) | (c == rc1);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] =
            mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    fetchA(st, 1, ra1);
    fetchB(st, 1, rb1);
    copy(dst, valid, 0, src);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] =
            mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    copy(dst, valid, 1, src);
    __builtin_amdgcn_sched_barrier(0);
    res_mfma(POS, ron, ra0, 0);
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(dst, valid, 2, src);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kHasNext) {
      // 3 of this chunk's copies and the 4 of the previous one may stay in flight
      if (late) WAIT_KEEP(23); else WAIT_KEEP(7);
      fetchA(next, 0, ra0);
      fetchB(next, 0, rb0);
    }
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(dst, valid, 3, src);
    __builtin_amdgcn_sched_barrier(0);
    res_mfma(POS, ron, ra1, 1);
    post(c);
  };

  UnitPos cur = unit_pos(t);
  fill_table(cur, 0);
  __syncthreads();
  set_copy_unit(cur, 0);
  dma(0, st0, true);
  dma(1, st1, 1 < nk);
  dma(2, st2, 2 < nk);

  bool first_unit = true;
  const std::integral_constant<bool, true> kFirst;
  const std::integral_constant<bool, false> kNext;
  for (;;) {
    const bool has_next = t + Gx < cnt;
    UnitPos nx = cur;
    if (has_next) nx = unit_pos(t + Gx);
    cur_su = cur.su;
    rc0 = a.residual ? res_chunk(0) : -1;
    rc1 = a.residual ? res_chunk(1) : -1;
    // The unit's first chunk starts the accumulators (FIRST) when there are more than four
    // chunks; with four, the last group is the first one and they are cleared beforehand.
    if (nk4 == 4) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = zero16;
    }

    // Every chunk is exactly 4 copies per wave, every copy is issued unconditionally and every
    // epilogue issues exactly 16 stores per wave, so the waits below are exact: at a chunk
    // boundary the two newer chunks stay in flight, and after the first unit the previous
    // epilogue's stores too, until chunk 3 (issued after them) is awaited. The branches on
    // `late` are uniform.
    const bool late = !first_unit;
    if (late) WAIT_KEEP(24); else WAIT_KEEP(8);
    first_unit = false;
    if (has_next) fill_table(nx, bf ^ 1);   // its readers come after later barriers
    fetchA(st0, 0, ra0);
    fetchB(st0, 0, rb0);
    if (nk4 > 4) {
      compute_pipe(kFirst, Pos<0>{}, st0, 0, 3, st3, 3 < nk, st1, late);
      compute_pipe(kNext, Pos<1>{}, st1, 1, 4, st0, 4 < nk, st2, late);
      compute_pipe(kNext, Pos<2>{}, st2, 2, 5, st1, 5 < nk, st3, false);
      compute_pipe(kNext, Pos<3>{}, st3, 3, 6, st2, 6 < nk, st0, false);
      for (int kc = 4; kc + 4 < nk4; kc += 4) {
        compute_pipe(kNext, Pos<0>{}, st0, kc, kc + 3, st3, kc + 3 < nk, st1, false);
        compute_pipe(kNext, Pos<1>{}, st1, kc + 1, kc + 4, st0, kc + 4 < nk, st2, false);
        compute_pipe(kNext, Pos<2>{}, st2, kc + 2, kc + 5, st1, kc + 5 < nk, st3, false);
        compute_pipe(kNext, Pos<3>{}, st3, kc + 3, kc + 6, st2, kc + 6 < nk, st0, false);
      }
    }
    {
      // last four chunks; the next unit's first three are copied meanwhile
      const int kc = nk4 - 4;
      const bool late4 = late && nk4 == 4;
      compute_pipe(kNext, Pos<0>{}, st0, kc, kc + 3, st3, kc + 3 < nk, st1, late4);
      if (has_next) set_copy_unit(nx, bf ^ 1);
      compute_pipe(kNext, Pos<1>{}, st1, kc + 1, 0, st0, has_next, st2, late4);
      compute_pipe(kNext, Pos<2>{}, st2, kc + 2, 1, st1, has_next && 1 < nk, st3, false);
      compute_pipe(kNext, Pos<3>{}, st3, kc + 3, 2, st2, has_next && 2 < nk, nullptr, false);
    }

    // ---- epilogue through stage 3: wave w uses bytes 4096 w .. +4095, a [32 tokens][64
    // features] bf16 tile whose 16-byte piece c of row r sits at c ^ ((r >> 1) & 7). A wave
    // writes and reads back only its own tile, so after the first barrier (every wave is done
    // reading stage 3) it needs none. Round (nb, fh): token block nb, features 128 wm + 64 fh.
    const __amdgpu_buffer_rsrc_t outr = make_rsrc(a.xhat + cur.b * a.N * a.ld_out, (uint32_t)(a.N * a.ld_out * 2));
    lds_sync();
    uint8_t* const stg = st3 + wave * 4096;
    // write: row lane & 31, half lane >> 5, piece c at wofs ^ (c << 4); read: row 8 it + (lane >> 3),
    // piece lane & 7, at (rofs ^ ((it & 1) << 6)) + 1024 it (the row's swizzle is 4 (it & 1) + (lane >> 4))
    const uint32_t wofs = ((uint32_t)(lane & 31) * 128u + 8u * (uint32_t)(lane >> 5)) | ((uint32_t)((lane >> 1) & 7) << 4);
    const uint32_t rofs = (uint32_t)(lane >> 3) * 128u + ((uint32_t)((lane & 7) ^ (lane >> 4)) << 4);
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const float bv = s_bias[(cur.su * TU + wn * 64 + nb * 32 + (lane & 31)) & 511];
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float y = acc[2 * fh + h][nb][g * 4 + e] + bv;
              v[e] = kRelu ? fmaxf(y, 0.f) : y;
            }
            *reinterpret_cast<uint2*>(stg + (wofs ^ ((uint32_t)(4 * h + g) << 4))) =
                make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
          }
        }
        const int f = cur.f_base + wm * 128 + fh * 64 + (lane & 7) * 8;
#pragma unroll
        for (int it = 0; it < 4; ++it) {
          const uint4 v = lds_read16(stg, (rofs ^ ((uint32_t)(it & 1) << 6)) + (uint32_t)it * 1024u);
          const int s = cur.su * TU + wn * 64 + nb * 32 + it * 8 + (lane >> 3);
          const int64_t tok = (int64_t)cur.i * a.S + s;
          const bool ok = s < a.S && tok < a.N && f < a.d;
          buf_store16<2>(outr, ok ? (uint32_t)((tok * a.ld_out + f) * 2) : OOB, 0, v);   // non-temporal
        }
      }
    }
    if (!has_next) break;
    t += Gx;
    cur = nx;
    bf ^= 1;
  }
  wait_vmem();   // the zero-filled copies issued past the last unit land before the exit
}

}  // namespace unit

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
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  // At least one 256 x 256 unit per CU: the persistent kernel; otherwise the tiled one, whose
  // smaller tiles keep more CUs busy. The persistent kernel keeps a unit's block table in one
  // lane per block, so it takes k + 1 <= 64 (the tiled kernel any k).
  const int64_t units = B * p.n_s * ((S + unit::TU - 1) / unit::TU) * p.f_tiles;
  if (units >= cus && k + 1 <= unit::kMaxBlocks) {
    p.s_tiles = (S + unit::TU - 1) / unit::TU;
    p.tiles = units;
    // chunks per block as a constant for the common split lengths
    const bool relu = epi.act != 0;
    if (S == 256) {
      if (relu) hipLaunchKernelGGL((unit::compress_unit_kernel<8, true>), dim3((unsigned)cus), dim3(512), 0, stream, p);
      else hipLaunchKernelGGL((unit::compress_unit_kernel<8, false>), dim3((unsigned)cus), dim3(512), 0, stream, p);
    } else if (S == 512) {
      if (relu) hipLaunchKernelGGL((unit::compress_unit_kernel<16, true>), dim3((unsigned)cus), dim3(512), 0, stream, p);
      else hipLaunchKernelGGL((unit::compress_unit_kernel<16, false>), dim3((unsigned)cus), dim3(512), 0, stream, p);
    } else {
      if (relu) hipLaunchKernelGGL((unit::compress_unit_kernel<0, true>), dim3((unsigned)cus), dim3(512), 0, stream, p);
      else hipLaunchKernelGGL((unit::compress_unit_kernel<0, false>), dim3((unsigned)cus), dim3(512), 0, stream, p);
    }
    return hipGetLastError();
  }
  p.tiles = B * p.n_s * p.s_tiles * p.f_tiles;
  hipLaunchKernelGGL(compress_bf16_kernel, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
