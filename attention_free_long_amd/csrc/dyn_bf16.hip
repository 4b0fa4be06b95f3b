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
//  2. O^T[f][p] = sum_q Z^T[f][q] G[q][p]: Z^T is read from LDS tiles of [128 q][128 f]
//     (S <= 256) or [64 q][256 f] (S <= 512) by the LDS transpose read, in the same q order;
//     each result lane owns token p and four
//     consecutive features, scaled by 1 / (r_p + eps). G is rounded to bf16 for this product
//     and r_p is summed from the rounded values, so the applied weights sum to r_p / (r_p + eps).
// Two kernels below: one 8-wave workgroup per split for S <= 256, four 4-wave workgroups per
// split (128 tokens p each) for S <= 512.
#include "avey_common.h"
#include "launch.h"

namespace avey {

namespace {

struct DynParams {
  const uint16_t* z;
  uint16_t* out;
  int64_t N, ld_z, ld_out, tiles;
  int m_t, S, n_s, pgroups;
  // S <= 256 kernel: splits full .. tiles - 1 (the last, partial wave of the grid) are each
  // shared by fsplit workgroups, which all compute the split's G and take consecutive ranges of
  // its phase-2 feature tiles; the fsplit workgroups of one split have ids fsplit NXCD apart
  // (the same XCD), so that their repeated phase-1 reads meet in its L2. fsplit = 1: none.
  int64_t full;
  int fsplit;
  // S = 64 and 128 (ring kernel): a workgroup takes 256 / S consecutive splits (S above is then
  // 256 and n_s counts the groups) and mixes tokens p, q only when p >> gshift == q >> gshift;
  // otherwise gshift is 8 and seg == S.
  int seg, gshift;
  float eps;
  LayerEpi epi;
};

// Bias of token position p (0 without a bias), loaded before any copy is issued and forced to
// complete there, so that no load but the copies is outstanding in the pipelined loops.
__device__ __forceinline__ float layer_bias(const LayerEpi& e, int p, bool p_ok) {
  float bv = 0.f;
  if (e.bias && p_ok) bv = e.bias[p];
  asm volatile("" : "+v"(bv));
  return bv;
}

// Row normalisation (LayerEpi::norm). Four cosines G_pq of row p, q = q0 .. q0 + 3, become the
// weights the second GEMM uses, rounded to bf16 (two packed pairs); stat accumulates what the
// row's scale is computed from, over the rounded weights: their sum (sum, softmax) or the sum
// of their squares (rms). Softmax weights are exp(G_pq) for valid q and 0 for padding q.
__device__ __forceinline__ void g_weights(float g0, float g1, float g2, float g3, int q0, int nvalid, int norm,
                                          uint32_t& lo, uint32_t& hi, float& stat, bool keep = true) {
  if (!keep) g0 = g1 = g2 = g3 = 0.f;   // q0 .. q0 + 3 belong to another split than p
  if (norm == kNormSoftmax) {
    g0 = keep && q0 + 0 < nvalid ? __expf(g0) : 0.f;
    g1 = keep && q0 + 1 < nvalid ? __expf(g1) : 0.f;
    g2 = keep && q0 + 2 < nvalid ? __expf(g2) : 0.f;
    g3 = keep && q0 + 3 < nvalid ? __expf(g3) : 0.f;
  }
  lo = pack_bf16(g0, g1);
  hi = pack_bf16(g2, g3);
  const float r0 = bf16lo(lo), r1 = bf16hi(lo), r2 = bf16lo(hi), r3 = bf16hi(hi);
  stat += norm == kNormRms ? (r0 * r0 + r1 * r1) + (r2 * r2 + r3 * r3) : (r0 + r1) + (r2 + r3);
}

// Scale of row p from its statistic: 1 / (sum + eps) (eq. 6), 1 / sum (softmax),
// 1 / sqrt(mean square + eps) over the nvalid tokens (rms), 1 (none).
__device__ __forceinline__ float row_scale(int norm, float stat, float eps, int nvalid) {
  if (norm == kNormSum) return 1.0f / (stat + eps);
  if (norm == kNormSoftmax) return 1.0f / stat;
  if (norm == kNormRms) return 1.0f / sqrtf(stat / (float)nvalid + eps);
  return 1.0f;
}

__device__ __forceinline__ float layer_out(float v, float scale, float bv, bool relu) {
  const float y = fmaf(v, scale, bv);
  return relu ? fmaxf(y, 0.f) : y;
}
template <bool kRelu>
__device__ __forceinline__ float layer_out(float v, float scale, float bv) {
  const float y = fmaf(v, scale, bv);
  return kRelu ? fmaxf(y, 0.f) : y;
}

// ---------------------------------------------------------------------------------------------
// S <= 256: one 8-wave workgroup per split, both GEMMs fed by one 4-stage ring of 32 KiB
// direct-copy stages (three chunks in flight while one is multiplied).
//   Phase 1, chunk kc: Z rows q = 0..255 x features 64 kc .. +63 (128-byte LDS rows). Wave w
//   owns p = 32 w .. 32 w + 31: C1[q][p] over all 256 q (8 MFMA blocks); the squared norms of
//   its p rows come from the B fragments it reads anyway.
//   Phase 2, chunk (ft, qh): Z rows q = 128 qh .. +127 x features 128 ft .. +127 (256-byte LDS
//   rows), read as Z^T fragments by the LDS transpose read, times the G fragments the wave
//   holds in registers: O^T[f][p] for 128 features x its 32 p, two chunks per feature tile.
// The phase-2 chunks stream without waiting for phase 1's result: only their products do.
// In both phases a wave reads the next k-step's fragments while the current one's MFMAs run,
// which the 128-feature tiles leave registers for (G alone takes 64 per lane).
namespace ring {

constexpr int QR = 256;                 // q rows per split (padded)
constexpr int STAGE = QR * ROWB;        // 32 KiB: phase 1 chunk (256 x 64 features)
constexpr int ZB = 512;                 // S <= 512 kernel, phase 2 LDS row: 256 features
constexpr int FT = 256;                 // S <= 512 kernel, phase 2 features per tile
constexpr int ZR = 256;                 // S <= 256 kernel, phase 2 LDS row: 128 features
constexpr int FR = 128;                 // S <= 256 kernel, phase 2 features per tile

__device__ __forceinline__ uint2 lds_read_tr8(const uint8_t* base, uint32_t off) {
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
  const bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + off));
  return __builtin_bit_cast(uint2, v);
}

#define DYN_WAIT_KEEP(n) asm volatile("s_waitcnt vmcnt(" #n ") lgkmcnt(0)\n\ts_barrier" ::: "memory")

// A copy's offset is computed on every lane and then selected (OOB for the lanes that load
// zeros): under a branch around it, every copy split the K loop into another basic block.
__device__ __forceinline__ uint32_t sel_off(bool ok, uint32_t o) {
  asm volatile("" : "+v"(o));
  return ok ? o : OOB;
}

template <bool kRelu>
__global__ void __launch_bounds__(512, 1) dyn_ring_kernel(DynParams a) {
  __shared__ __align__(16) uint8_t st0[STAGE], st1[STAGE], st2[STAGE], st3[STAGE];
  __shared__ float s_sq[QR];
  __shared__ __align__(16) float s_rn[QR];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);

  const int nft_all = (a.m_t + FR - 1) / FR;     // phase-2 feature tiles of a split
  int64_t split;
  int ft0 = 0, nft = nft_all;                     // this workgroup's phase-2 feature tiles
  if ((int64_t)blockIdx.x < a.full) {
    split = xcd_remap(blockIdx.x, a.full);
  } else {
    // 32-bit arithmetic (the grid is below 2^32) on wave-uniform values, kept in scalar registers
    const uint32_t j = blockIdx.x - (uint32_t)a.full, l = j / NXCD, f = (uint32_t)a.fsplit;
    const uint32_t grp = (uint32_t)uniform((int)(l / f)), k = l - grp * f;
    split = a.full + (int64_t)grp * NXCD + j % NXCD;
    if (split >= a.tiles) return;                 // the grid's tail rounded up to whole XCD rounds
    ft0 = uniform((int)(k * (uint32_t)nft_all / f));
    nft = uniform((int)((k + 1) * (uint32_t)nft_all / f)) - ft0;
  }
  const int64_t b = split / a.n_s;
  const int i = (int)(split % a.n_s);
  const int64_t base = (int64_t)i * a.S;
  const int valid_rows = (int)min((int64_t)a.S, a.N - base);
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z + b * a.N * a.ld_z, (uint32_t)(a.N * a.ld_z * 2));
  // Phase 2 addresses features from this workgroup's first tile: its reads and stores go through
  // descriptors whose base is moved by ft0 tiles, against m_loc features left.
  const int m_loc = a.m_t - ft0 * FR;
  const __amdgpu_buffer_rsrc_t zr2 =
      make_rsrc(a.z + b * a.N * a.ld_z + ft0 * FR, (uint32_t)((a.N * a.ld_z - ft0 * FR) * 2));
  const int p = wave * 32 + (lane & 31);          // this lane's output token (in the workgroup's rows)
  const bool p_ok = p < valid_rows;
  const int pseg = p >> a.gshift;                 // p's split among the workgroup's (0 unless grouped)
  const float bv = layer_bias(a.epi, p - (pseg << a.gshift), p_ok);   // bias of p's position in its split
  const int nk1 = (a.m_t + KC - 1) / KC;          // phase-1 chunks of 64 features (last partial)
  const int nk1p = (nk1 + 3) / 4 * 4;             // padded with zero chunks to a multiple of 4

  // ---- copies: 4 per wave per chunk, zeros when !valid or out of range. The two phases have
  // separate copy routines, chosen at compile time at every call site: a run-time branch
  // between them would join control flow around the copies, after which the compiler drains
  // all copies before the next LDS read.
  auto copy1 = [&](int c, uint8_t* st, bool valid, int n) __attribute__((always_inline)) {
    // rows 32 w + 8 n .. + 7 of chunk c, 128 bytes each; lane -> row (ln >> 3), position (ln & 7);
    // 16-byte pieces past m_t (the last chunk when m_t % 64 != 0) load zeros
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int row = wave * 32 + n * 8 + (ln >> 3);
    const uint32_t pc = (uint32_t)((ln & 7) ^ (int)swz<SWZ_ROW>(row));
    const bool ok = valid && c < nk1 && row < valid_rows && 8 * (int)pc < a.m_t - c * KC;
    dma16(zr, st + (wave * 32 + n * 8) * ROWB, sel_off(ok, (uint32_t)((base + row) * a.ld_z * 2) + 16u * pc),
          (uint32_t)c * KC * 2u);
  };
  auto copy2 = [&](int c2, uint8_t* st, bool valid, int n) __attribute__((always_inline)) {
    // rows 16 w + 4 n .. + 3 (256 bytes each) of q half qh, f tile ft; LDS 32-byte slot s of row
    // t holds the row's 32-byte piece s ^ 2 (t & 3)
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // Phase 2 walks the workgroup's feature tiles from the last one down: phase 1 read the
    // split's last features most recently, so the first tiles' copies can still meet them in
    // the L2. Logical tile c2 >> 1 is feature tile nft - 1 - (c2 >> 1) (the epilogue maps it the
    // same way).
    const int ft = nft - 1 - (c2 >> 1), qh = c2 & 1;
    const int t = wave * 16 + n * 4 + (ln >> 4);
    const int q = qh * 128 + t;
    const int pp = ln & 15;
    const int pc = (pp >> 1) ^ (2 * (t & 3));
    const int f = ft * FR + pc * 16 + (pp & 1) * 8;
    const bool ok = valid && c2 < 2 * nft && q < valid_rows && f < m_loc;
    dma16(zr2, st + (wave * 16 + n * 4) * ZR, sel_off(ok, (uint32_t)(((base + q) * a.ld_z + f) * 2)), 0);
  };

  // ---- phase 1
  uint32_t fq[4], fp[4];
  frag_offsets<SWZ_ROW>(fq, 0, lane);
  frag_offsets<SWZ_ROW>(fp, wave * 32, lane);
  f32x16 acc1[8];
#pragma unroll
  for (int qb = 0; qb < 8; ++qb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc1[qb][v] = 0.f;
  float sq = 0.f;
  // Fragments of the k-step being multiplied: ra for the 8 q blocks, rb for this wave's p block.
  // The next k-step's are read in two halves, each right after the MFMAs that last read those
  // registers are issued, so that the reads run under the other half's MFMAs. A chunk's last
  // k-step reads the next chunk's first one the same way, after the wait and barrier for that
  // chunk, which therefore sit between the two MFMA halves.
  // The fragment offsets are laundered through an empty asm at each read, so that the stage
  // base is added there: hoisted, the sums for every stage would be long-lived registers.
  uint4 ra[8], rb, rbn;
  auto read1 = [&](const uint8_t* st, int ks, int h) __attribute__((always_inline)) {
    if (h == 0) {
      uint32_t o = fp[ks];
      asm volatile("" : "+v"(o));
      rbn = lds_read16(st, o);
    }
    uint32_t o = fq[ks];
    asm volatile("" : "+v"(o));
#pragma unroll
    for (int qb = 4 * h; qb < 4 * h + 4; ++qb) ra[qb] = lds_read16(st, o + qb * 32 * ROWB);
  };
  // One chunk of MFMAs from stage st, whose first k-step is in ra / rb; issue(ks) issues the
  // ks-th copy of a later chunk; next is the following chunk's stage, or nullptr for none: its
  // type decides at compile time (a run-time test of the stage pointer, which the compiler cannot
  // prove non-null, put a branch into every chunk).
  auto compute1 = [&](const uint8_t* st, auto&& issue, auto next) __attribute__((always_inline)) {
    constexpr bool kHasNext = !std::is_same_v<decltype(next), std::nullptr_t>;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      sq = sumsq8(rb, sq);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) acc1[qb] = mfma32(as_bf16x8(ra[qb]), as_bf16x8(rb), acc1[qb]);
      if (ks < 3) {
        read1(st, ks + 1, 0);
      } else if constexpr (kHasNext) {
        DYN_WAIT_KEEP(7);   // 3 of this chunk's copies and the 4 of the previous one may stay in flight
        read1(next, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int qb = 4; qb < 8; ++qb) acc1[qb] = mfma32(as_bf16x8(ra[qb]), as_bf16x8(rb), acc1[qb]);
      if (ks < 3) {
        read1(st, ks + 1, 1);
      } else if constexpr (kHasNext) {
        read1(next, 0, 1);
      }
      rb = rbn;
      issue(ks);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  auto c1 = [&](int c, uint8_t* dst) { return [=, &copy1](int n) { copy1(c, dst, true, n); }; };
  auto c2 = [&](int c, uint8_t* dst) { return [=, &copy2](int n) { copy2(c, dst, true, n); }; };

  for (int n = 0; n < 4; ++n) copy1(0, st0, true, n);
  for (int n = 0; n < 4; ++n) copy1(1, st1, true, n);
  for (int n = 0; n < 4; ++n) copy1(2, st2, true, n);
  DYN_WAIT_KEEP(8);
  read1(st0, 0, 0);
  read1(st0, 0, 1);
  rb = rbn;
  for (int kc = 0; kc + 4 < nk1p; kc += 4) {
    compute1(st0, c1(kc + 3, st3), st1);
    compute1(st1, c1(kc + 4, st0), st2);
    compute1(st2, c1(kc + 5, st1), st3);
    compute1(st3, c1(kc + 6, st2), st0);
  }
  {
    // last four phase-1 chunks; the first three phase-2 chunks are copied meanwhile
    const int kc = nk1p - 4;
    compute1(st0, c1(kc + 3, st3), st1);
    compute1(st1, c2(0, st0), st2);
    compute1(st2, c2(1, st1), st3);
    compute1(st3, c2(2, st2), nullptr);
  }

  // ---- norms, G (bf16) as phase-2 B fragments, r_p from the rounded values
  {
    const float t = sq + __shfl_xor(sq, 32);    // the two lane halves hold the two k-halves
    if (lane < 32) s_sq[wave * 32 + lane] = t;
  }
  lds_sync();
  if (tid < QR) {
    const float ss = s_sq[tid];
    s_rn[tid] = (tid < valid_rows && ss > 0.f) ? 1.0f / sqrtf(ss) : 0.f;
  }
  lds_sync();
  uint4 gfrag[8][2];
  float inv;
  {
    const float rnp = s_rn[wave * 32 + (lane & 31)];
    float r = 0.f;
#pragma unroll
    for (int qb = 0; qb < 8; ++qb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q0 = qb * 32 + s2 * 16 + h * 8 + (lane >> 5) * 4;   // rows of v = 8 s2 + 4 h + 0..3
          const float4 rq = *reinterpret_cast<const float4*>(&s_rn[q0]);
          const int v0 = s2 * 8 + h * 4;
          g_weights(acc1[qb][v0 + 0] * rq.x * rnp, acc1[qb][v0 + 1] * rq.y * rnp, acc1[qb][v0 + 2] * rq.z * rnp,
                    acc1[qb][v0 + 3] * rq.w * rnp, q0, valid_rows, a.epi.norm, pk[2 * h + 0], pk[2 * h + 1], r,
                    (q0 >> a.gshift) == pseg);
        }
        gfrag[qb][s2] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
    r += __shfl_xor(r, 32);
    // valid tokens of p's split (the RMS mean runs over them)
    inv = row_scale(a.epi.norm, r, a.eps, min(a.seg, valid_rows - (pseg << a.gshift)));
  }

  // ---- phase 2. G fragment (qb, s2) of lane half h holds q = 32 qb + 16 s2 + {4h .. 4h+3,
  // 8+4h .. 8+4h+3}; the Z^T fragments are read with the same q order (two transpose reads:
  // tokens +4h and +8+4h), features 32 fb + (l & 31). The offset of block fb in a chunk row is
  // ((2 fb + g1) ^ 2 s2x) * 32 + 8 (l & 3), so the fragment offset is offZ0 ^ (fb << 6) (the
  // row, lane and g1 terms fill other bits): one register for all four blocks.
  uint32_t offZ0;
  {
    const int s2x = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    const uint32_t row = (uint32_t)(4 * (lane >> 5) + ((lane & 15) >> 2)) * ZR;
    offZ0 = row + (uint32_t)((g1 << 5) | (s2x << 6)) + 8u * (lane & 3);
  }
  f32x16 acc2[4];
  const f32x16 zero16 = {};
  uint4 rz[4], rzn[4];   // Z^T fragments of the k-step being multiplied and of the next one
  auto read2 = [&](const uint8_t* st, int ks) __attribute__((always_inline)) {   // token rows 16 ks .. +15
    uint32_t o0 = offZ0;
    asm volatile("" : "+v"(o0));
    const uint32_t tok = (uint32_t)(16 * ks) * ZR;
#pragma unroll
    for (int fb = 0; fb < 4; ++fb) {
      const uint32_t o = o0 ^ ((uint32_t)fb << 6);
      const uint2 lo = lds_read_tr8(st, o + tok);
      const uint2 hi = lds_read_tr8(st, o + tok + 8 * ZR);
      rzn[fb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  // One chunk (q half qh of a feature tile) from stage st, whose first k-step is in rzn; the
  // copies of phase-2 chunk cnext into dst go out at k-steps 0, 2, 4 and 6. With next, the
  // following chunk's wait and barrier sit between the two MFMA halves of the last k-step, and
  // its first k-step is read there: 4 copies of the chunk after it and the 4 of this chunk may
  // stay in flight, and (after_epi) the 8 stores of the epilogue before this chunk.
  auto compute2 = [&](const uint8_t* st, auto qh_tag, int cnext, uint8_t* dst, auto next,
                      auto after_epi) __attribute__((always_inline)) {
    constexpr int qh = decltype(qh_tag)::value;
    constexpr bool kHasNext = !std::is_same_v<decltype(next), std::nullptr_t>;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
#pragma unroll
      for (int fb = 0; fb < 4; ++fb) rz[fb] = rzn[fb];
      const uint4 gb = gfrag[4 * qh + (ks >> 1)][ks & 1];
      // the tile's first k-step starts the accumulators from an inline zero
      const bool first = qh == 0 && ks == 0;
      if (ks < 7) read2(st, ks + 1);
#pragma unroll
      for (int fb = 0; fb < 2; ++fb) acc2[fb] = mfma32(as_bf16x8(rz[fb]), as_bf16x8(gb), first ? zero16 : acc2[fb]);
      if constexpr (kHasNext) {
        if (ks == 7) {
          if constexpr (decltype(after_epi)::value) DYN_WAIT_KEEP(16); else DYN_WAIT_KEEP(8);
          read2(next, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int fb = 2; fb < 4; ++fb) acc2[fb] = mfma32(as_bf16x8(rz[fb]), as_bf16x8(gb), first ? zero16 : acc2[fb]);
      if ((ks & 1) == 0) copy2(cnext, dst, true, ks >> 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Epilogue of feature tile ft, staged through stage sst (the tile's second chunk, done) in two
  // rounds of 64 features: each lane writes its 4-feature groups into a [256 tokens][64 features]
  // bf16 tile (16-byte piece c of row t at c ^ ((t >> 1) & 7)), then 8 lanes per token store
  // whole 128-byte row pieces (scattered 8-byte stores would cost a write request per lane, and
  // 64-byte pieces measured slower). A wave writes and reads only its own 32 rows, so after the
  // first barrier (every wave is done reading the stage) it needs none. Every wave issues exactly
  // 8 stores per tile (lanes past the split or past m_t store out of range), which the next
  // tile's waits allow for: the stores drain under the MFMAs instead of holding up the next tile.
  const __amdgpu_buffer_rsrc_t outr =
      make_rsrc(a.out + b * a.N * a.ld_out + ft0 * FR, (uint32_t)((a.N * a.ld_out - ft0 * FR) * 2));
  // write: row p, piece c at wofs ^ (c << 4); read: row 32 w + 8 it + (lane >> 3), piece lane & 7,
  // at rofs ^ ((it & 1) << 6) + 1024 it (the row's swizzle is 4 (it & 1) + (lane >> 4))
  const uint32_t wofs = ((uint32_t)p * 128u + 8u * (uint32_t)(lane >> 5)) | ((uint32_t)((p >> 1) & 7) << 4);
  const uint32_t rofs = (uint32_t)(wave * 32 + (lane >> 3)) * 128u + ((uint32_t)((lane & 7) ^ (lane >> 4)) << 4);
  uint32_t srow[4];   // byte offset of each read row's token in the output, OOB past the split
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int t = wave * 32 + it * 8 + (lane >> 3);
    srow[it] = t < valid_rows ? (uint32_t)((base + t) * a.ld_out * 2) : OOB;
  }
  auto epilogue = [&](int ft, uint8_t* sst) __attribute__((always_inline)) {
    lds_sync();   // every wave is done reading the stage
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        const int fb = 2 * rr + fh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = pack_bf16(layer_out<kRelu>(acc2[fb][g * 4 + 0], inv, bv),
                                        layer_out<kRelu>(acc2[fb][g * 4 + 1], inv, bv));
          const uint32_t hi = pack_bf16(layer_out<kRelu>(acc2[fb][g * 4 + 2], inv, bv),
                                        layer_out<kRelu>(acc2[fb][g * 4 + 3], inv, bv));
          *reinterpret_cast<uint2*>(sst + (wofs ^ ((uint32_t)(4 * fh + g) << 4))) = make_uint2(lo, hi);
        }
      }
      const int f = (nft - 1 - ft) * FR + rr * 64 + (lane & 7) * 8;
      const bool fok = f < m_loc;
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const uint4 v = lds_read16(sst, (rofs ^ ((uint32_t)(it & 1) << 6)) + (uint32_t)it * 1024u);
        buf_store16<2>(outr, fok ? srow[it] + (uint32_t)f * 2u : OOB, 0, v);   // non-temporal
      }
    }
  };
  // Feature tile ft: chunks 2 ft (stage sa) and 2 ft + 1 (stage sb); the copies issued meanwhile
  // are those of chunks 2 ft + 3 (into sd) and 2 ft + 4 (into sa). Its first chunk is complete
  // once at most 8 newer copies are outstanding, and after an epilogue its 8 stores as well
  // (16). The epilogue comes between two tiles, so a tile's first k-step is read after that
  // wait, not ahead.
  auto tile = [&](int ft, uint8_t* sa, uint8_t* sb, uint8_t* sd, auto after_epi) __attribute__((always_inline)) {
    const std::integral_constant<int, 0> kQ0;
    const std::integral_constant<int, 1> kQ1;
    const std::integral_constant<bool, false> kNoStores;
    if constexpr (decltype(after_epi)::value) DYN_WAIT_KEEP(16); else DYN_WAIT_KEEP(8);
    read2(sa, 0);
    compute2(sa, kQ0, 2 * ft + 3, sd, sb, after_epi);
    compute2(sb, kQ1, 2 * ft + 4, sa, nullptr, kNoStores);
    epilogue(ft, sb);
  };
  const std::integral_constant<bool, true> kAfterEpi;
  tile(0, st0, st1, st3, std::integral_constant<bool, false>{});
  int ft = 1;
  for (; ft + 1 < nft; ft += 2) {
    tile(ft, st2, st3, st1, kAfterEpi);
    tile(ft + 1, st0, st1, st3, kAfterEpi);
  }
  if (ft < nft) tile(ft, st2, st3, st1, kAfterEpi);
  wait_vmem();   // the copies issued past the last chunk and the last stores complete before the exit
}

// ---------------------------------------------------------------------------------------------
// 256 < S <= 512: a split's G row block for 128 tokens p, over all 512 q, fills the register
// file of a wave per 32 p (16 accumulator blocks), so a workgroup of 4 waves (one per SIMD)
// takes 128 p and a split takes 4 workgroups, each reading the whole split.
//   Phase 1, chunk kc: Z rows q = 0..511 x features 64 kc .. +63, as two halves of 256 rows in
//   separate LDS objects (two stages of 64 KiB, one chunk in flight).
//   Phase 2: the 4-stage ring of the S <= 256 kernel, chunk (ft, qc) = Z rows 64 qc .. +63 x
//   features 256 ft .. +255 (8 chunks per feature tile, 8 copies per wave per chunk), read as
//   Z^T fragments by the LDS transpose read against the G fragments the wave holds.
constexpr int QR5 = 512;
constexpr int HALF = 256 * ROWB;        // 32 KiB: 256 rows of a phase-1 chunk, or a phase-2 stage

__global__ void __launch_bounds__(256, 1) dyn512_kernel(DynParams a) {
  __shared__ __align__(16) uint8_t st0[HALF], st1[HALF], st2[HALF], st3[HALF];
  __shared__ float s_sq[QR5];
  __shared__ __align__(16) float s_rn[QR5];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = uniform(tid >> 6);

  const int64_t L = xcd_remap(blockIdx.x, a.tiles);
  const int pg = (int)(L % a.pgroups);
  const int64_t split = L / a.pgroups;
  const int64_t b = split / a.n_s;
  const int i = (int)(split % a.n_s);
  const int64_t base = (int64_t)i * a.S;
  const int nvalid = (int)min((int64_t)a.S, a.N - base);   // valid tokens of the split
  const __amdgpu_buffer_rsrc_t zr = make_rsrc(a.z + b * a.N * a.ld_z, (uint32_t)(a.N * a.ld_z * 2));
  const int nk = (a.m_t + KC - 1) / KC;           // phase-1 chunks (the last one partial)

  // ---- phase 1: C1[q][p] for all 512 q and this wave's 32 p. Wave w copies rows 64 w .. +63 of
  // each half of a chunk (8 copies of 8 rows per half), so that every copy has a fixed LDS
  // object as its destination (with a selected one, the compiler would wait for the copies in
  // flight before reading either half).
  const int prow0 = pg * 128 + wave * 32;          // this wave's first p (split-local)
  const int p = prow0 + (lane & 31);               // this lane's output token
  const bool relu = a.epi.act != 0;
  const float bv = layer_bias(a.epi, p, p < nvalid);
  uint32_t offZ[16];
#pragma unroll
  for (int n = 0; n < 16; ++n) {
    const int row = (n >> 3) * 256 + wave * 64 + (n & 7) * 8 + (lane >> 3);
    const uint32_t c = (uint32_t)((lane & 7) ^ (int)swz<SWZ_ROW>(row));
    offZ[n] = row < nvalid ? (uint32_t)((base + row) * a.ld_z * 2) + 16u * c : OOB;
  }
  // fragment offsets within a 256-row half (the swizzle repeats every 16 rows)
  uint32_t fq[4], fp[4], fn[4];
  frag_offsets<SWZ_ROW>(fq, 0, lane);
  frag_offsets<SWZ_ROW>(fp, prow0 & 255, lane);
  frag_offsets<SWZ_ROW>(fn, wave * 64, lane);
  const bool p_hi = prow0 >= 256;

  f32x16 acc1[16];
#pragma unroll
  for (int qb = 0; qb < 16; ++qb)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc1[qb][v] = 0.f;
  // squared norms (k-halves) of rows 256 (j >> 1) + 64 w + 32 (j & 1) + (l & 31)
  float sq[4] = {0.f, 0.f, 0.f, 0.f};

  // Chunk kc; the 16-byte pieces past m_t (the last chunk when m_t % 64 != 0) load zeros: the
  // piece of copy n is (l & 7) ^ ((4 (n & 1) + (l >> 4)) & 7), the swizzle of its row.
  auto dma1 = [&](int kc, uint8_t* lo, uint8_t* hi) {
    const int lim = a.m_t - kc * KC;
    auto off = [&](int n) {
      const int c = (lane & 7) ^ ((4 * (n & 1) + (lane >> 4)) & 7);
      return offZ[n] | ((uint32_t)(8 * c >= lim) << 31);
    };
#pragma unroll
    for (int n = 0; n < 8; ++n) dma16(zr, lo + (wave * 64 + n * 8) * ROWB, off(n), (uint32_t)kc * KC * 2);
#pragma unroll
    for (int n = 0; n < 8; ++n) dma16(zr, hi + (wave * 64 + n * 8) * ROWB, off(8 + n), (uint32_t)kc * KC * 2);
  };
  // Every LDS read names its object (a read through a selected pointer would also wait for
  // the copies in flight): the p fragment is read from both halves and selected. The next
  // k-step's fragments are read before this one's MFMAs.
  struct Frags1 {
    uint4 q[16], p;
  };
  auto fetch1 = [&](const uint8_t* lo, const uint8_t* hi, int ks, Frags1& f) {
    const uint4 rlo = lds_read16(lo, fp[ks]), rhi = lds_read16(hi, fp[ks]);
    f.p = p_hi ? rhi : rlo;
#pragma unroll
    for (int qb = 0; qb < 16; ++qb) f.q[qb] = lds_read16(qb < 8 ? lo : hi, fq[ks] + (qb & 7) * 32 * ROWB);
  };
  auto compute1 = [&](const uint8_t* lo, const uint8_t* hi) {
    Frags1 f0, f1;
    fetch1(lo, hi, 0, f0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frags1& cur = (ks & 1) ? f1 : f0;
      Frags1& nxt = (ks & 1) ? f0 : f1;
      if (ks < 3) fetch1(lo, hi, ks + 1, nxt);
#pragma unroll
      for (int j = 0; j < 4; ++j) sq[j] = sumsq8(lds_read16(j < 2 ? lo : hi, fn[ks] + (j & 1) * 32 * ROWB), sq[j]);
#pragma unroll
      for (int qb = 0; qb < 16; ++qb) acc1[qb] = mfma32(as_bf16x8(cur.q[qb]), as_bf16x8(cur.p), acc1[qb]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  dma1(0, st0, st1);
  wait_vmem();
  __syncthreads();
  int kc = 0;
  for (; kc + 2 <= nk; kc += 2) {
    dma1(kc + 1, st2, st3);
    compute1(st0, st1);
    wait_vmem();
    __syncthreads();
    if (kc + 2 < nk) dma1(kc + 2, st0, st1);
    compute1(st2, st3);
    wait_vmem();
    __syncthreads();
  }
  if (kc < nk) {
    compute1(st0, st1);
    __syncthreads();
  }

  // ---- norms, G (bf16) as phase-2 B fragments, r_p from the rounded values
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const float t = sq[j] + __shfl_xor(sq[j], 32);   // the two lane halves hold the two k-halves
    if (lane < 32) s_sq[(j >> 1) * 256 + wave * 64 + (j & 1) * 32 + lane] = t;
  }
  __syncthreads();
  for (int q = tid; q < QR5; q += 256) {
    const float ss = s_sq[q];
    s_rn[q] = (q < nvalid && ss > 0.f) ? 1.0f / sqrtf(ss) : 0.f;
  }
  __syncthreads();
  uint4 gfrag[16][2];
  float inv;
  {
    const float rnp = s_rn[p];
    float r = 0.f;
#pragma unroll
    for (int qb = 0; qb < 16; ++qb) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        uint32_t pk[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int q0 = qb * 32 + s2 * 16 + h * 8 + (lane >> 5) * 4;   // rows of v = 8 s2 + 4 h + 0..3
          const float4 rq = *reinterpret_cast<const float4*>(&s_rn[q0]);
          const int v0 = s2 * 8 + h * 4;
          g_weights(acc1[qb][v0 + 0] * rq.x * rnp, acc1[qb][v0 + 1] * rq.y * rnp, acc1[qb][v0 + 2] * rq.z * rnp,
                    acc1[qb][v0 + 3] * rq.w * rnp, q0, nvalid, a.epi.norm, pk[2 * h + 0], pk[2 * h + 1], r);
        }
        gfrag[qb][s2] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      }
    }
    r += __shfl_xor(r, 32);
    inv = row_scale(a.epi.norm, r, a.eps, nvalid);
  }

  // ---- phase 2
  const int nft = (a.m_t + FT - 1) / FT;
  const int total = 8 * nft;
  // copy n (0..7) of chunk c2 into stage st: rows 16 w + 2 n, + 1 (512 bytes each); 32-byte
  // piece (p >> 1) ^ 2 (t & 3) of row t
  auto copy2 = [&](int c2, uint8_t* st, int n) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int ft = c2 >> 3, qc = c2 & 7;
    const int t = wave * 16 + n * 2 + (ln >> 5);
    const int q = qc * 64 + t;
    const int pp = ln & 31;
    const int pc = (pp >> 1) ^ (2 * (t & 3));
    const int f = ft * FT + pc * 16 + (pp & 1) * 8;
    const bool ok = (c2 < total) & (q < nvalid) & (f < a.m_t);   // no short-circuit: no branch
    dma16(zr, st + (wave * 16 + n * 2) * ZB, sel_off(ok, (uint32_t)(((base + q) * a.ld_z + f) * 2)), 0);
  };
  uint32_t offZ2[8];
  {
    const int s2x = (lane >> 2) & 3, g1 = (lane >> 4) & 1;
    const uint32_t row = (uint32_t)(4 * (lane >> 5) + ((lane & 15) >> 2)) * ZB;
#pragma unroll
    for (int fb = 0; fb < 8; ++fb)
      offZ2[fb] = row + (uint32_t)(((2 * fb + g1) ^ (2 * s2x)) << 5) + 8u * (lane & 3);
  }
  f32x16 acc2[8];
  const f32x16 zero16 = {};
  // Z^T fragments of k-step ks (q = 32 (ks >> 1) + 16 (ks & 1) + the G fragment's order)
  auto fetch2 = [&](const uint8_t* st, int ks, uint4 (&ra)[8]) {
    const uint32_t tok = (uint32_t)(32 * (ks >> 1) + 16 * (ks & 1)) * ZB;
#pragma unroll
    for (int fb = 0; fb < 8; ++fb) {
      const uint2 lo = lds_read_tr8(st, offZ2[fb] + tok);
      const uint2 hi = lds_read_tr8(st, offZ2[fb] + tok + 8 * ZB);
      ra[fb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
  };
  // Chunk qc of a feature tile from stage st; the 8 copies of chunk cnext go into dst meanwhile.
  // With one wave per SIMD nothing else hides the fragment reads, so the next k-step's are
  // issued before this one's MFMAs.
  auto compute2 = [&](const uint8_t* st, auto qc_tag, int cnext, uint8_t* dst) {
    constexpr int qc = decltype(qc_tag)::value;
    uint4 ra0[8], ra1[8];
    fetch2(st, 0, ra0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      uint4 (&cur)[8] = (ks & 1) ? ra1 : ra0;
      uint4 (&nxt)[8] = (ks & 1) ? ra0 : ra1;
      if (ks < 3) fetch2(st, ks + 1, nxt);
      const uint4 gb = gfrag[2 * qc + (ks >> 1)][ks & 1];
      const bool first = qc == 0 && ks == 0;   // the tile's first k-step starts from zero
#pragma unroll
      for (int fb = 0; fb < 8; ++fb) acc2[fb] = mfma32(as_bf16x8(cur[fb]), as_bf16x8(gb), first ? zero16 : acc2[fb]);
      copy2(cnext, dst, 2 * ks);
      copy2(cnext, dst, 2 * ks + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // Epilogue of feature tile ft through stage 3 in four rounds of 64 features ([128 tokens][64
  // features] bf16, 16-byte piece c of row t at c ^ ((t >> 1) & 7)), stored as whole 128-byte
  // row pieces by 8 lanes per token. A wave writes and reads back only its own 32 rows, so after
  // the first barrier (every wave is done reading stage 3) it needs none. Every wave issues
  // exactly 16 stores per tile (lanes past the split or past m_t store out of range), which the
  // next tile's first three copy waits allow for.
  const __amdgpu_buffer_rsrc_t outr = make_rsrc(a.out + b * a.N * a.ld_out, (uint32_t)(a.N * a.ld_out * 2));
  const int pl = wave * 32 + (lane & 31);          // this lane's token within the workgroup
  auto epilogue = [&](int ft) {
    lds_sync();   // every wave is done reading stage 3
    const uint32_t rowo = (uint32_t)pl * 128u + 8u * (uint32_t)(lane >> 5);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
#pragma unroll
      for (int fh = 0; fh < 2; ++fh) {
        const int fb = 2 * rr + fh;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t lo = pack_bf16(layer_out(acc2[fb][g * 4 + 0], inv, bv, relu),
                                        layer_out(acc2[fb][g * 4 + 1], inv, bv, relu));
          const uint32_t hi = pack_bf16(layer_out(acc2[fb][g * 4 + 2], inv, bv, relu),
                                        layer_out(acc2[fb][g * 4 + 3], inv, bv, relu));
          const uint32_t pc = (uint32_t)(4 * fh + g) ^ (uint32_t)((pl >> 1) & 7);
          *reinterpret_cast<uint2*>(st3 + rowo + (pc << 4)) = make_uint2(lo, hi);
        }
      }
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const int t = wave * 32 + it * 8 + (lane >> 3);
        const int pp = lane & 7;
        const uint4 v = lds_read16(st3, (uint32_t)t * 128u + ((uint32_t)(pp ^ ((t >> 1) & 7)) << 4));
        const int f = ft * FT + rr * 64 + pp * 8;
        const int tp = pg * 128 + t;
        const bool ok = tp < nvalid && f < a.m_t;
        buf_store16<2>(outr, ok ? (uint32_t)(((base + tp) * a.ld_out + f) * 2) : OOB, 0, v);   // non-temporal
      }
    }
  };
  // The phase-1 stages are free (the barriers above); chunks 0..2 go into stages 0..2. Before
  // chunk c: its 8 copies are complete in every wave (the 16 newer ones may stay in flight, and
  // after an epilogue for chunks c0 .. c0 + 2 its 16 stores as well; the branch on ft is uniform).
  for (int n = 0; n < 8; ++n) copy2(0, st0, n);
  for (int n = 0; n < 8; ++n) copy2(1, st1, n);
  for (int n = 0; n < 8; ++n) copy2(2, st2, n);
  for (int ft = 0; ft < nft; ++ft) {
    const int c0 = 8 * ft;
    if (ft) DYN_WAIT_KEEP(32); else DYN_WAIT_KEEP(16);
    compute2(st0, std::integral_constant<int, 0>{}, c0 + 3, st3);
    if (ft) DYN_WAIT_KEEP(32); else DYN_WAIT_KEEP(16);
    compute2(st1, std::integral_constant<int, 1>{}, c0 + 4, st0);
    if (ft) DYN_WAIT_KEEP(32); else DYN_WAIT_KEEP(16);
    compute2(st2, std::integral_constant<int, 2>{}, c0 + 5, st1);
    DYN_WAIT_KEEP(16);
    compute2(st3, std::integral_constant<int, 3>{}, c0 + 6, st2);
    DYN_WAIT_KEEP(16);
    compute2(st0, std::integral_constant<int, 4>{}, c0 + 7, st3);
    DYN_WAIT_KEEP(16);
    compute2(st1, std::integral_constant<int, 5>{}, c0 + 8, st0);
    DYN_WAIT_KEEP(16);
    compute2(st2, std::integral_constant<int, 6>{}, c0 + 9, st1);
    DYN_WAIT_KEEP(16);
    compute2(st3, std::integral_constant<int, 7>{}, c0 + 10, st2);
    epilogue(ft);
  }
  wait_vmem();   // the copies issued past the last chunk and the last stores complete before the exit
}

}  // namespace ring

int64_t device_cus() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return cus;
}

}  // namespace

hipError_t launch_dyn_bf16(const uint16_t* z, int64_t B, int64_t N, int m_t, int64_t ld_z, int S, float eps,
                           uint16_t* out, int64_t ld_out, hipStream_t stream, LayerEpi epi) {
  DynParams p;
  p.z = z; p.out = out;
  p.N = N; p.ld_z = ld_z; p.ld_out = ld_out;
  p.m_t = m_t; p.S = S; p.eps = eps;
  p.epi = epi;
  p.seg = S;
  p.gshift = 8;
  if (S == 64 || S == 128) {   // 256 / S splits per workgroup
    p.S = 256;
    p.gshift = S == 64 ? 6 : 7;
  }
  p.n_s = (int)((N + p.S - 1) / p.S);
  p.tiles = B * p.n_s;
  p.pgroups = 1;
  p.full = p.tiles;
  p.fsplit = 1;
  if (p.S <= 256) {
    // One workgroup per CU at a time. When the grid's last wave would leave half the CUs or
    // more idle, its r splits are shared by f = min(CUs / r, feature tiles, 4) workgroups each.
    const int64_t cus = device_cus();
    const int64_t waves = (p.tiles + cus - 1) / cus, r = p.tiles - (waves - 1) * cus;
    const int64_t f = min(min(cus / r, (int64_t)(m_t + ring::FR - 1) / ring::FR), (int64_t)4);
    int64_t grid = p.tiles;
    if (f >= 2) {
      p.full = (waves - 1) * cus;
      p.fsplit = (int)f;
      grid = p.full + (r + NXCD - 1) / NXCD * NXCD * f;
    }
    if (epi.act != 0) hipLaunchKernelGGL(ring::dyn_ring_kernel<true>, dim3((unsigned)grid), dim3(512), 0, stream, p);
    else hipLaunchKernelGGL(ring::dyn_ring_kernel<false>, dim3((unsigned)grid), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
  p.pgroups = (S + 127) / 128;   // workgroups of 128 tokens p per split
  p.tiles *= p.pgroups;
  hipLaunchKernelGGL(ring::dyn512_kernel, dim3((unsigned)p.tiles), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace avey
