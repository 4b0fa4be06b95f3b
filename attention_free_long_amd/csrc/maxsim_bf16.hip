// All-pairs split MaxSim on bf16 MFMA (gfx950).
//
// MaxSim relevance of candidate split j to target split i is the sum over the tokens t of i of
// the largest cosine between x_t and any token u of j (paperlayer.ai "Avey-B" summary,
// section 3; papernotes.org Avey-B note, 方法详解/整体框架). With n_t = N(x_t) the L2-normalised
// token (papernotes.org Avey-B note, 关键设计 2) and C = X_i X_j^T the tile of dot products,
// cos(x_t, x_u) = C_tu rn_t rn_u with rn = 1 / |x| (0 for a zero token), and both directions of
// the pair come from one tile:
//   score(i <- j) = sum_t rn_t max_u C_tu rn_u          (row direction)
//   score(j <- i) = sum_u rn_u max_t C_tu rn_t          (column direction)
// Each unordered pair i < j is computed once, and no token-by-token similarity leaves the chip.
//
// Two operand sources, one kernel template:
//   * row-major (kRow): the caller's X as it is ([B, N, d], row stride ld). Every wave sums the
//     squares of one 32-row block of each operand from the MFMA fragments it reads anyway, so
//     the norms of the unit's 512 tokens are on chip when the K loop ends, and the epilogue
//     scales each direction's candidates before taking maxima. Nothing but the scores is
//     written to memory.
//   * packed: a copy of N(x) that prepare.hip wrote split by split in chunk planes of 32
//     features ([B][n_s][nk][S][32] bf16): the tile holds the cosines themselves, and every copy
//     instruction reads 1 KiB of contiguous memory.
//
// Units are 256 target rows x 256 candidate rows (one per pair at S <= 256, four at S <= 512).
// At S = 64 and 128 a unit side is instead a group of 256 / S consecutive splits (kG of them):
// 256 consecutive tokens, which is how the row-major X and the workspace (packed in blocks of
// 256 rows at these S) already lie, so the K loop and the copies are the same. Each unit then
// serves every pair between its two groups (including the pairs inside one group, on the
// diagonal units), and the epilogue keeps one maximum per split: columns of one split are whole
// waves (64 or 128 columns), rows of one split whole 32-row blocks.
// One workgroup of 8 waves per CU (2 per SIMD), in a 2 x 4 grid: each wave owns 128 x 64 of the
// fp32 accumulator (8 MFMA 32x32x16 blocks). Features stream through a 4-stage LDS ring in
// chunks of 32 by direct global -> LDS copies, three chunks in flight while one is multiplied
// (the copies of a chunk are issued between the MFMA groups of the chunk being multiplied, and
// the wait for the next chunk comes before the last group, whose MFMAs hide the next chunk's
// first fragment reads);
// the next unit's first three chunks are copied while the current one finishes and during its
// epilogue.
//
// Persistent grid: workgroups are dealt to the 8 XCDs round-robin; each XCD owns one contiguous
// range of pair tiles, walked in bands of 8 target splits, so that the target operands of the
// concurrently resident tiles stay in the XCD's L2 while candidates stream past: the 32 tiles an
// XCD runs at a time are 8 targets x 4 candidates, each candidate read by 8 of them (bands of 8
// measured 1-2% faster than bands of 4 at 96K tokens, the same at 32K; 16 was slower).
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
  const uint16_t* x;    // kRow: X [B, N, d] row stride ld; packed: N(x) [B][n_s][nk][S][32]
  int64_t ld;           // kRow: row stride of X in elements
  int64_t N;
  int d, S, n_s;
  int nk;               // chunks of 32 features (the last one partial when d % 32 != 0)
  int q;                // 256-row blocks per split
  int pairs;            // unordered pairs per sequence
  int64_t tiles;        // B * pairs
  float* scores;
  int n_out;            // splits per sequence in the score matrix (n_s, or the real count when grouped)
};

// Unordered pair p of one sequence -> (i, j), i < j. Pairs come in bands of H = BAND target
// splits: the H (H - 1) / 2 pairs inside the band, then the band x later-splits rectangle in
// candidate-major order. A full band I holds H n_s - H^2 I - H (H + 1) / 2 pairs, so
// P(I) = I (H n_s - H / 2) - (H^2 / 2) I^2 pairs precede it.
constexpr int BAND = 8;
__device__ void decode_pair(int p, int n_s, int& i, int& j) {
  constexpr int H = BAND;
  const int nfull = n_s / H;
  auto P = [&](int I) -> long long {
    return (long long)I * ((long long)H * n_s - H / 2) - (long long)(H * H / 2) * I * I;
  };
  const long long pfull = P(nfull);
  int i0, h;
  long long rem;
  if (p < pfull) {
    const double bq = (double)H * n_s - H / 2;
    int I = (int)((bq - sqrt(bq * bq - 2.0 * H * H * (double)p)) / (double)(H * H));
    I = max(0, min(I, nfull - 1));
    while (I + 1 < nfull && P(I + 1) <= p) ++I;
    while (I > 0 && P(I) > p) --I;
    i0 = H * I;
    h = H;
    rem = p - P(I);
  } else {
    i0 = H * nfull;
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

// kG: splits per unit side (1, or 256 / S at S = 64 and 128, where a.S is 256 and a.n_s counts
// the groups).
template <bool kRow, bool kTail, int kG>
__global__ void __launch_bounds__(512, 1) maxsim_bf16_kernel(MaxsimParams a) {
  static_assert(kG == 1 || kG == 2 || kG == 4, "splits per unit side");
  // One LDS object per stage (target block, then candidate block): the compiler tracks copies
  // per object, so reads of one stage do not wait for copies into another. Stage 3 doubles as
  // the epilogue's row-max scratch.
  __shared__ __align__(16) uint8_t st0[2 * T * RB], st1[2 * T * RB], st2[2 * T * RB], st3[2 * T * RB];
  __shared__ __align__(16) float s_biA[T];   // per target row: 0, or -inf for a padding token
  __shared__ __align__(16) float s_biB[T];   // per candidate row
  __shared__ __align__(16) float s_rnA[T];   // kRow: per target row 1 / |x_t| (0 for a zero token)
  __shared__ __align__(16) float s_rnB[T];   // kRow: per candidate row
  __shared__ float s_ssA[2 * T], s_ssB[2 * T];   // kRow: running sums of squares, [k-half][row]
  // column maxima per row segment (the two row halves; at kG = 4 the four 64-row splits) x lane half
  __shared__ float s_cm[kG == 4 ? 4 : 2][2][T];
  __shared__ float s_colmax[2 * T];          // running column maxima over target blocks (S = 512)
  __shared__ float s_red[8];
  __shared__ float s_redg[8][kG];            // grouped units: per wave, one sum per split of the other side

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

  const int nk = a.nk;
  // Accumulator slot s of the wave holds its target-row block blkA(s) (32 rows), slot u its
  // candidate-row block blkB(u). kRow rotates the slots so that slot 0 is the block whose token
  // norms this wave sums: target block wn of its row half, candidate block wm of its column
  // quarter; the eight waves cover each operand's 256 rows once.
  const int rotA = kRow ? wn : 0, rotB = kRow ? wm : 0;
  auto blkA = [&](int s_) { return (s_ + rotA) & 3; };
  auto blkB = [&](int u_) { return (u_ + rotB) & 1; };
  uint32_t fa[2], fb[2];   // fragment offsets of the two k-steps of a chunk, block 0
#pragma unroll
  for (int ks = 0; ks < 2; ++ks) {
    const int ra = wm * 128 + (lane & 31), rb = wn * 64 + (lane & 31);
    fa[ks] = (uint32_t)ra * RB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(ra)) << 4);
    fb[ks] = (uint32_t)rb * RB + ((((uint32_t)(2 * ks + (lane >> 5))) ^ sw4(rb)) << 4);
  }
  // Fragment offset of slot s at k-step ks. kRow rebuilds the rotated target-block offsets at
  // each read (the base laundered through an empty asm): held, they would take 8 more long-lived
  // registers and spill. The 4 candidate-block offsets are held.
  auto offA = [&](int ks, int s_) {
    uint32_t o = fa[ks];
    if (kRow) asm volatile("" : "+v"(o));
    return o + (uint32_t)blkA(s_) * 32 * RB;
  };
  auto offB = [&](int ks, int u_) {
    uint32_t o = fb[ks];
    return o + (uint32_t)blkB(u_) * 32 * RB;
  };

  // Tile t of this workgroup is pair (xs + t) % pairs of sequence (xs + t) / pairs. The
  // division runs once; each later tile advances the pair index by Gx and carries into the
  // sequence (scalar work), so that no 64-bit division, whose constants take vector registers,
  // sits in the unit loop. The pair decode runs on the vector unit (double-precision square
  // root); its results are wave-uniform and are moved to scalar registers, so that everything
  // derived from them (block offsets, limits, the descriptor base) stays out of the vector
  // register file.
  auto tile_at = [&](int b, int p) {
    Unit u;
    u.b = b;
    int i, j;
    if (kG == 1) {
      decode_pair(p, a.n_s, i, j);
    } else {
      // pairs of groups I <= J: the unordered pairs I < J' of n_s + 1 with J = J' - 1
      decode_pair(p, a.n_s + 1, i, j);
      j -= 1;
    }
    u.i = uniform(i);
    u.j = uniform(j);
    u.ua = 0;
    u.ub = 0;
    return u;
  };
  int tb = (int)((xs + t) / a.pairs);   // sequence and pair index of tile t
  int tp = (int)((xs + t) % a.pairs);

  // Copy addressing: a descriptor over the unit's sequence, the byte offsets of its two blocks'
  // first rows in chunk 0, the bytes from one token row to the next (rowB) and from one chunk to
  // the next (chunkB). Packed: rows are 64 bytes apart inside a chunk plane of S rows; kRow:
  // rows are ld * 2 bytes apart and a chunk is the next 64 bytes of the row.
  const uint16_t* xbase = a.x;   // the copy unit's sequence
  uint32_t xbytes = 0;
  int limA = 0, limB = 0;        // valid (non-padding) rows of the unit's blocks
  uint32_t pbA = 0, pbB = 0;
  const uint32_t rowB = kRow ? (uint32_t)(a.ld * 2) : (uint32_t)RB;
  const uint32_t chunkB = kRow ? (uint32_t)RB : (uint32_t)a.S * RB;
  // Each lane's copy offsets of the copy unit (block base, row, piece; kRow: the row clamped to
  // the block's last valid row), held, so that a copy costs one select; with kTail a lane's
  // pieces past d also depend on the chunk, and the offsets are built per copy.
  uint32_t hoA[2] = {0u, 0u}, hoB[2] = {0u, 0u};
  auto set_unit = [&](const Unit& u) {
    const int64_t seq = kRow ? a.N * a.ld : (int64_t)a.n_s * a.nk * a.S * KH;
    xbase = a.x + u.b * seq;
    xbytes = (uint32_t)(seq * 2);
    limA = (int)min((int64_t)min(a.S - u.ua * T, T), a.N - ((int64_t)u.i * a.S + u.ua * T));
    limB = (int)min((int64_t)min(a.S - u.ub * T, T), a.N - ((int64_t)u.j * a.S + u.ub * T));
    if (kRow) {
      pbA = (uint32_t)(((int64_t)u.i * a.S + u.ua * T) * rowB);
      pbB = (uint32_t)(((int64_t)u.j * a.S + u.ub * T) * rowB);
      // each lane's offsets of copies n = 0, 1 of both blocks, held for the unit (chunk 0)
      const int sub = lane >> 2, pc = (lane & 3) ^ ((sub >> 2) & 3);
#pragma unroll
      for (int n = 0; n < (kTail ? 0 : 2); ++n) {
        const int r0 = wave * 32 + n * 16;
        hoA[n] = pbA + (uint32_t)(min(r0 + sub, limA - 1) * (int)rowB) + 16u * (uint32_t)pc;
        hoB[n] = pbB + (uint32_t)(min(r0 + sub, limB - 1) * (int)rowB) + 16u * (uint32_t)pc;
      }
    } else {
      pbA = (uint32_t)((int64_t)u.i * a.nk * a.S * RB + u.ua * T * RB);
      pbB = (uint32_t)((int64_t)u.j * a.nk * a.S * RB + u.ub * T * RB);
      const int sub = lane >> 2, pc = (lane & 3) ^ ((sub >> 2) & 3);
#pragma unroll
      for (int n = 0; n < 2; ++n) {
        const uint32_t lo = (uint32_t)(wave * 32 + n * 16 + sub) * RB + 16u * (uint32_t)pc;
        hoA[n] = pbA + lo;
        hoB[n] = pbB + lo;
      }
    }
  };
  // Lane l of a copy lands at LDS row r0 + (l >> 2), position l & 3, so it fetches the logical
  // 16-byte piece pc = (l & 3) ^ sw4(row) of its row: features 8 pc .. 8 pc + 7 of the chunk.
  // kRow: an LDS row past the block's valid rows is filled from the block's last valid row, so
  // that padding rows repeat a real token (neither maximum changes; the sums skip them) and no
  // row t >= N is read; with d % 32 != 0 (kTail) the pieces past d load zeros. Lane terms are
  // recomputed per copy (laundered through an empty asm so they are not hoisted into long-lived
  // registers).
  auto src_off = [&](bool ok, uint32_t pb, int lim, int r0, int sub, int pc) {
    uint32_t o;
    if (kRow) {
      const int r = max(min(min(r0 + sub, lim - 1), 255), -256);
      o = pb + (uint32_t)(r * (int)(rowB & 0x3fffffu)) + 16u * (uint32_t)pc;
    } else {
      o = pb + (uint32_t)(r0 + sub) * rowB + 16u * (uint32_t)pc;
    }
    asm volatile("" : "+v"(o));
    return ok ? o : OOB;
  };
  auto lane_terms = [&](int& sub, int& pc) {
    sub = lane >> 2;
    asm volatile("" : "+v"(sub));
    pc = (lane & 3) ^ ((sub >> 2) & 3);
  };
  auto live = [&](int kc, int pc, bool valid) {
    return kTail ? (valid && 8 * pc < a.d - kc * KH) : valid;
  };
  // Chunk kc of the current copy unit into stage st: wave w copies rows [32w, 32w + 32) of both
  // blocks, 16 rows per instruction, 4 instructions. With valid == false every lane loads zeros.
  auto dma = [&](int kc, uint8_t* st, bool valid) {
    int sub, pc;
    lane_terms(sub, pc);
    const bool ok = live(kc, pc, valid);
    const uint32_t kb = (uint32_t)kc * chunkB;
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int r0 = wave * 32 + n * 16;
      const __amdgpu_buffer_rsrc_t xr = make_rsrc_uniform(xbase, xbytes);
      if (!kTail) {
        dma16(xr, st + r0 * RB, ok ? hoA[n] : OOB, kb);
        dma16(xr, st + T * RB + r0 * RB, ok ? hoB[n] : OOB, kb);
      } else {
        dma16(xr, st + r0 * RB, src_off(ok, pbA, limA, r0, sub, pc), kb);
        dma16(xr, st + T * RB + r0 * RB, src_off(ok, pbB, limB, r0, sub, pc), kb);
      }
    }
  };

  f32x16 acc[4][2];
  // Fragments of k-step 0 (ra0, rb0) and 1 (ra1, rb1) of the chunk being multiplied, by slot.
  uint4 ra0[4], rb0[2], ra1[4], rb1[2];
  auto fetch0 = [&](const uint8_t* st) {
#pragma unroll
    for (int s_ = 0; s_ < 4; ++s_) ra0[s_] = lds_read16(st, offA(0, s_));
#pragma unroll
    for (int u_ = 0; u_ < 2; ++u_) rb0[u_] = lds_read16(st + T * RB, offB(0, u_));
  };
  auto fetch1 = [&](const uint8_t* st) {
#pragma unroll
    for (int s_ = 0; s_ < 4; ++s_) ra1[s_] = lds_read16(st, offA(1, s_));
#pragma unroll
    for (int u_ = 0; u_ < 2; ++u_) rb1[u_] = lds_read16(st + T * RB, offB(1, u_));
  };
  // kRow reads each k-step's fragments in two halves, target blocks 0-1 with the candidate
  // blocks, then target blocks 2-3 once the previous k-step's MFMAs that read those registers
  // are issued: at most 32 fragment registers are live instead of 40, which leaves room for the
  // norm sums and the scale registers of the epilogue.
  auto fetch_lo = [&](uint4 (&ra)[4], uint4 (&rb)[2], int ks, const uint8_t* st) {
#pragma unroll
    for (int s_ = 0; s_ < 2; ++s_) ra[s_] = lds_read16(st, offA(ks, s_));
#pragma unroll
    for (int u_ = 0; u_ < 2; ++u_) rb[u_] = lds_read16(st + T * RB, offB(ks, u_));
  };
  auto fetch_hi = [&](uint4 (&ra)[4], int ks, const uint8_t* st) {
#pragma unroll
    for (int s_ = 2; s_ < 4; ++s_) ra[s_] = lds_read16(st, offA(ks, s_));
  };
  // kRow: sums of squares of this wave's norm rows (slot 0 of each operand). Each lane sums the 8
  // features of its k-half over the unit's chunks into tA / tB and writes the total to its entry
  // of s_ssA[half][row] at the unit's last chunk (each lane owns one entry: no atomics). The
  // epilogue adds the two halves and clears them.
  float tA = 0.f, tB = 0.f;
  auto ss_slot = [&]() {
    int o = (lane >> 5) * T + (lane & 31);
    asm volatile("" : "+v"(o));
    return o;
  };
  if (kRow) {
    const int o = ss_slot();
    s_ssA[o + wm * 128 + wn * 32] = 0.f;
    s_ssB[o + wn * 64 + wm * 32] = 0.f;
  }
  // One chunk from stage st whose k-step-0 fragments are already in ra0 / rb0; the 4 copies of
  // chunk kc into dst go between the MFMA groups. With a next stage the next chunk's wait and
  // barrier come before the last MFMA group, and its k-step-0 fragments are read under it; the
  // unit's last chunk passes nullptr, whose type tells the two apart at compile time (a run-time
  // test of the stage pointer stays in the loop, the compiler not knowing it non-null).
  // FIRST: the unit's first chunk, whose k-step-0 MFMAs start the accumulators from zero (an
  // inline constant) instead of reading them, so that nothing has to clear them.
  const f32x16 zero16 = {};
  auto compute_pipe = [&](auto FIRST, const uint8_t* st, int kc, uint8_t* dst, bool valid, auto next) {
    constexpr bool kHasNext = !std::is_same_v<decltype(next), std::nullptr_t>;
    int sub, pc;
    lane_terms(sub, pc);
    const bool ok = live(kc, pc, valid);
    const uint32_t kb = (uint32_t)kc * chunkB;
    auto copy = [&](int ks, int h) {
      const int r0 = wave * 32 + ks * 16;
      // the descriptor is rebuilt from the first lane at each copy: carried across the loop it
      // is taken as per-lane, and every copy through it became a loop over distinct values
      const __amdgpu_buffer_rsrc_t xr = make_rsrc_uniform(xbase, xbytes);
      if (!kTail) {
        uint32_t o = h == 0 ? hoA[ks] : hoB[ks];
        asm volatile("" : "+v"(o));   // a select, not a branch
        if (h == 0) dma16(xr, dst + r0 * RB, ok ? o : OOB, kb);
        else dma16(xr, dst + T * RB + r0 * RB, ok ? o : OOB, kb);
      } else {
        if (h == 0) dma16(xr, dst + r0 * RB, src_off(ok, pbA, limA, r0, sub, pc), kb);
        else dma16(xr, dst + T * RB + r0 * RB, src_off(ok, pbB, limB, r0, sub, pc), kb);
      }
    };
    if (kRow) {   // before the MFMAs, which stay the fragments' last readers
      tA = sumsq8(ra0[0], tA);
      tB = sumsq8(rb0[0], tB);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    if (kRow) {
      fetch_lo(ra1, rb1, 1, st);
    } else {
      fetch1(st);
    }
    copy(0, 0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
        acc[mb][nb] = mfma32(as_bf16x8(ra0[mb]), as_bf16x8(rb0[nb]), FIRST.value ? zero16 : acc[mb][nb]);
    if (kRow) fetch_hi(ra1, 1, st);
    copy(0, 1);
    __builtin_amdgcn_sched_barrier(0);
    if (kRow) {
      tA = sumsq8(ra1[0], tA);
      tB = sumsq8(rb1[0], tB);
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    copy(1, 0);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kHasNext) {
      // 3 of this chunk's copies and the 4 of the previous one may stay in flight
      WAIT_KEEP(7);
      if (kRow) {
        fetch_lo(ra0, rb0, 0, next);
      } else {
        fetch0(next);
      }
    } else if (kRow) {
      const int so = ss_slot();
      s_ssA[so + wm * 128 + wn * 32] += tA;
      s_ssB[so + wn * 64 + wm * 32] += tB;
    }
#pragma unroll
    for (int mb = 2; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) acc[mb][nb] = mfma32(as_bf16x8(ra1[mb]), as_bf16x8(rb1[nb]), acc[mb][nb]);
    if constexpr (kHasNext) {
      if (kRow) fetch_hi(ra0, 0, next);
    }
    copy(1, 1);
    __builtin_amdgcn_sched_barrier(0);
  };

  // Thread tid < 256 owns target row tid of the unit, thread tid >= 256 candidate column
  // tid - 256; part accumulates its share of the pair's score.
  const bool is_row = tid < T;
  const int own = tid & (T - 1);
  float rmax = 0.f, part = 0.f;

  Unit cur = tile_at(tb, tp);
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
    int np_next = 0;   // pair index of the next tile, when the unit after this is one
    if (cur.ub + 1 < a.q) {
      nx.ub = cur.ub + 1;
    } else if (cur.ua + 1 < a.q) {
      nx.ua = cur.ua + 1;
      nx.ub = 0;
    } else if (t + Gx < cnt) {
      // tp + Gx, carried into the sequence, without forming a value past pairs
      int step = Gx, nb = tb;
      np_next = tp;
      while (step >= a.pairs - np_next) {
        step -= a.pairs - np_next;
        np_next = 0;
        ++nb;
      }
      np_next += step;
      nx = tile_at(nb, np_next);
    } else {
      has_next = false;
    }
    if (kRow) {
      tA = 0.f;
      tB = 0.f;
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
    if (!kRow) {
      if (is_row) s_biA[own] = valid ? 0.f : -INFINITY;
      else s_biB[own] = valid ? 0.f : -INFINITY;
    }
    if (kRow) {
      // the token norms of this wave's rows from its own LDS sums (the two k-halves); the sums
      // restart at zero for the next unit
      if (lane < 32) {
        const int ia = wm * 128 + wn * 32 + lane, ib = wn * 64 + wm * 32 + lane;
        const float sa = s_ssA[ia] + s_ssA[T + ia], sb = s_ssB[ib] + s_ssB[T + ib];
        s_ssA[ia] = 0.f;
        s_ssA[T + ia] = 0.f;
        s_ssB[ib] = 0.f;
        s_ssB[T + ib] = 0.f;
        s_rnA[ia] = sa > 0.f ? 1.0f / sqrtf(sa) : 0.f;
        s_rnB[ib] = sb > 0.f ? 1.0f / sqrtf(sb) : 0.f;
      }
    }
    lds_sync();   // also: every wave is done reading stage 3

    // One pass over the accumulators, both directions:
    //   column u: max over this wave's 128 rows -> cm, then across the two row halves
    //   row t:    max over this wave's 64 columns -> scratch [128 rows][8 lane quads] per wave
    // A two-step transposing max across the 4 lanes of a quad leaves lane q with row e = q of
    // each group of 4 rows, so each lane stores one value per group.
    const int q = lane & 3, par = lane & 1, hi2 = (lane >> 1) & 1;
    // per-lane scratch slot; kRow rebuilds it at each store (rotated block offsets, held for
    // every slot, would be long-lived registers)
    auto wscr_at = [&](int idx) {
      int o = wave * (128 * 8) + ((lane & 31) >> 2);
      if (kRow) asm volatile("" : "+v"(o));
      return reinterpret_cast<float*>(st3) + o + idx;
    };
    // column maxima over this wave's rows, per row segment: one (its 128 rows) unless kG = 4,
    // where its two 64-row halves are different splits
    constexpr int NH = kG == 4 ? 2 : 1;
    float cm[NH][2];
#pragma unroll
    for (int h = 0; h < NH; ++h) cm[h][0] = cm[h][1] = -INFINITY;
    auto reduce_store = [&](int ba, int g, const float (&m)[4]) {
      // step 1, lanes l and l ^ 1: the even lane keeps rows e = 0, 2, the odd lane e = 1, 3
      const float s0 = par ? m[0] : m[1], k0 = par ? m[1] : m[0];
      const float s1 = par ? m[2] : m[3], k1 = par ? m[3] : m[2];
      const float t0 = fmaxf(k0, __builtin_amdgcn_update_dpp(0.f, s0, 0xB1, 0xF, 0xF, false));
      const float t1 = fmaxf(k1, __builtin_amdgcn_update_dpp(0.f, s1, 0xB1, 0xF, 0xF, false));
      // step 2, lanes l and l ^ 2: keep row e = par (hi2 == 0) or e = par + 2 (hi2 == 1)
      const float s2 = hi2 ? t0 : t1, k2 = hi2 ? t1 : t0;
      const float f = fmaxf(k2, __builtin_amdgcn_update_dpp(0.f, s2, 0x4E, 0xF, 0xF, false));
      *wscr_at((ba * 32 + g * 8 + (lane >> 5) * 4 + q) * 8) = f;
    };
    // Accumulator element v of slot (s, u) in lane l: row blkA(s)*32 + 8(v >> 2) + 4(l >> 5) + (v & 3)
    // of the wave's rows, column blkB(u)*32 + (l & 31) of its columns.
    if (kRow) {
      // Padding rows and columns repeat a valid token, so no mask is needed. Column direction:
      // the accumulators are scaled in place by rn_t, C_tu rn_t, and maximised over this wave's
      // rows; row direction: the scaled values times rn_u are the cosines, maximised over this
      // wave's columns. At kG = 4 the column maxima are kept per slot and sorted into the two
      // row halves afterwards (the slots are rotated by wn).
      float cmS[kG == 4 ? 4 : 1][2];
#pragma unroll
      for (int s_ = 0; s_ < (kG == 4 ? 4 : 1); ++s_) cmS[s_][0] = cmS[s_][1] = -INFINITY;
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_) {
        int lo = (lane >> 5) * 4;
        asm volatile("" : "+v"(lo));
        const float* rnA_lane = s_rnA + wm * 128 + blkA(s_) * 32 + lo;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const float4 rs = *reinterpret_cast<const float4*>(rnA_lane + g * 8);
          const float rs4[4] = {rs.x, rs.y, rs.z, rs.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
#pragma unroll
            for (int u_ = 0; u_ < 2; ++u_) {
              acc[s_][u_][g * 4 + e] *= rs4[e];
              float& c = cmS[kG == 4 ? s_ : 0][u_];
              c = fmaxf(c, acc[s_][u_][g * 4 + e]);
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int u_ = 0; u_ < 2; ++u_) {
        if (kG == 4) {
#pragma unroll
          for (int s_ = 0; s_ < 4; ++s_) {
            const bool upper = ((s_ + rotA) & 2) != 0;   // block blkA(s_) lies in rows 64 .. 127
            cm[NH - 1][u_] = upper ? fmaxf(cm[NH - 1][u_], cmS[kG == 4 ? s_ : 0][u_]) : cm[NH - 1][u_];
            cm[0][u_] = upper ? cm[0][u_] : fmaxf(cm[0][u_], cmS[kG == 4 ? s_ : 0][u_]);
          }
        } else {
          cm[0][u_] = cmS[0][u_];
        }
      }
      float csc[2];
#pragma unroll
      for (int u_ = 0; u_ < 2; ++u_) csc[u_] = s_rnB[wn * 64 + blkB(u_) * 32 + (lane & 31)];
#pragma unroll
      for (int s_ = 0; s_ < 4; ++s_) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float m[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            m[e] = fmaxf(acc[s_][0][g * 4 + e] * csc[0], acc[s_][1][g * 4 + e] * csc[1]);
          reduce_store(blkA(s_), g, m);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    } else if (full) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float m[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float c0 = acc[mb][0][g * 4 + e], c1 = acc[mb][1][g * 4 + e];
            m[e] = fmaxf(c0, c1);
            cm[(mb >> 1) & (NH - 1)][0] = fmaxf(cm[(mb >> 1) & (NH - 1)][0], c0);
            cm[(mb >> 1) & (NH - 1)][1] = fmaxf(cm[(mb >> 1) & (NH - 1)][1], c1);
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
            cm[(mb >> 1) & (NH - 1)][0] = fmaxf(cm[(mb >> 1) & (NH - 1)][0], c0 + rb4[e]);
            cm[(mb >> 1) & (NH - 1)][1] = fmaxf(cm[(mb >> 1) & (NH - 1)][1], c1 + rb4[e]);
          }
          reduce_store(mb, g, m);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // both lane halves store their column maxima (the owner of the column takes the max of the
    // four), so no cross-lane exchange is needed here
#pragma unroll
    for (int h = 0; h < NH; ++h)
#pragma unroll
      for (int u_ = 0; u_ < 2; ++u_) s_cm[wm * NH + h][lane >> 5][wn * 64 + blkB(u_) * 32 + (lane & 31)] = cm[h][u_];
    lds_sync();
    if constexpr (kG == 1) {
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
        float cmv = fmaxf(fmaxf(s_cm[0][0][own], s_cm[0][1][own]), fmaxf(s_cm[1][0][own], s_cm[1][1][own]));
        if (!first_ua) cmv = fmaxf(cmv, s_colmax[cur.ub * T + own]);
        if (!last_ua) s_colmax[cur.ub * T + own] = cmv;
        else if (valid) part += kRow ? cmv * s_rnB[own] : cmv;
      }

      if (last_ua && last_ub) {
        // ---- scores of the pair; fixed reduction order (bitwise reproducible)
        // within each 16-lane row by DPP (lane ^ 1, lane ^ 2, then the mirrors l <-> 7 - l within
        // 8 lanes and l <-> 15 - l within 16), then the four row sums read from lanes 0, 16, 32 and
        // 48: no LDS round trip on this dependency chain
        float r = part;
        r += __builtin_amdgcn_update_dpp(0.f, r, 0xB1, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x4E, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x141, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x140, 0xF, 0xF, false);
        auto lane_f = [&](int l) {
          return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), l));
        };
        const float rs = ((lane_f(0) + lane_f(16)) + lane_f(32)) + lane_f(48);
        if (lane == 0) s_red[wave] = rs;
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
    } else {
      // ---- grouped unit: every pair between target split I kG + a and candidate split
      // J kG + b. Row owner t (target split a = t / S): one maximum per candidate split b, over
      // the quad maxima of the waves holding b's columns; column owner u (candidate split
      // b = u / S): one maximum per target split a. Sums over the S rows (columns) of one split
      // are per-wave DPP sums, then over the waves of the split, in a fixed order.
      constexpr int WPS = 4 / kG;   // waves (of 64 rows or columns) per split
      float pg[kG];
      if (is_row) {
        const int wr = own >> 7, rl = own & 127;
        const float* p = reinterpret_cast<const float*>(st3) + wr * (4 * 128 * 8) + rl * 8;
#pragma unroll
        for (int b_ = 0; b_ < kG; ++b_) {
          float m = -INFINITY;
#pragma unroll
          for (int w = b_ * WPS; w < (b_ + 1) * WPS; ++w) {
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              const int cc = ((c + (rl >> 3)) & 1) * 4;   // rotation: no bank conflicts
              const float4 u = *reinterpret_cast<const float4*>(p + w * (128 * 8) + cc);
              m = fmaxf(m, fmaxf(fmaxf(u.x, u.y), fmaxf(u.z, u.w)));
            }
          }
          pg[b_] = valid ? m : 0.f;
        }
      } else {
#pragma unroll
        for (int a_ = 0; a_ < kG; ++a_) {
          const float cmv = fmaxf(s_cm[a_][0][own], s_cm[a_][1][own]);
          pg[a_] = valid ? (kRow ? cmv * s_rnB[own] : cmv) : 0.f;
        }
      }
#pragma unroll
      for (int v = 0; v < kG; ++v) {
        float r = pg[v];
        r += __builtin_amdgcn_update_dpp(0.f, r, 0xB1, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x4E, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x141, 0xF, 0xF, false);
        r += __builtin_amdgcn_update_dpp(0.f, r, 0x140, 0xF, 0xF, false);
        auto lane_f = [&](int l) {
          return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, r), l));
        };
        const float rs = ((lane_f(0) + lane_f(16)) + lane_f(32)) + lane_f(48);
        if (lane == 0) s_redg[wave][v] = rs;
      }
      lds_sync();
      if (tid < kG * kG) {
        const int a_ = tid / kG, b_ = tid % kG;
        float tr = 0.f, tc = 0.f;
#pragma unroll
        for (int w = 0; w < WPS; ++w) {
          tr += s_redg[a_ * WPS + w][b_];        // rows of target split a_, maxima over b_
          tc += s_redg[4 + b_ * WPS + w][a_];    // columns of candidate split b_, maxima over a_
        }
        const int si = cur.i * kG + a_, sj = cur.j * kG + b_;
        if (si < a.n_out && sj < a.n_out) {
          float* sb = a.scores + cur.b * (int64_t)a.n_out * a.n_out;
          if (cur.i == cur.j) {
            // a diagonal unit: the row direction gives every ordered pair inside the group
            sb[(int64_t)si * a.n_out + sj] = a_ == b_ ? -INFINITY : tr;
          } else {
            sb[(int64_t)si * a.n_out + sj] = tr;
            sb[(int64_t)sj * a.n_out + si] = tc;
          }
        }
      }
    }

    if (!has_next) break;
    if (nx.ua == 0 && nx.ub == 0) {
      t += Gx;
      tb = (int)nx.b;
      tp = np_next;
    }
    cur = nx;
    lds_sync();   // this epilogue's LDS reads are done before stage 3 is refilled
  }
  wait_vmem();    // the zero-filled copies issued past the last unit land before the exit
}

// Splits per unit side: 256 / S at S = 64 and 128, else 1.
int group_of(int S) { return (S == 64 || S == 128) ? T / S : 1; }

MaxsimParams params(const uint16_t* x, int64_t ld, int64_t B, int64_t N, int d, int S, float* scores) {
  const int g = group_of(S);
  MaxsimParams p;
  p.x = x;
  p.ld = ld;
  p.N = N;
  p.d = d;
  p.S = S * g;                              // rows of a unit side: a split, or a group of splits
  p.n_s = (int)((N + p.S - 1) / p.S);
  p.n_out = (int)((N + S - 1) / S);
  p.nk = (d + KH - 1) / KH;
  p.q = (p.S + T - 1) / T;
  // unordered pairs of splits, or of groups with the diagonal (a group's own pairs)
  p.pairs = (int)(g == 1 ? (int64_t)p.n_s * (p.n_s - 1) / 2 : (int64_t)p.n_s * (p.n_s + 1) / 2);
  p.tiles = B * (int64_t)p.pairs;
  p.scores = scores;
  return p;
}

int64_t grid_for(int64_t tiles) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  return tiles < cus ? tiles : cus;
}

}  // namespace

// The kernel tracks a tile's sequence in 32 bits: batches beyond kMaxLaunchB sequences go out as
// several launches over consecutive slices of the batch.
constexpr int64_t kMaxLaunchB = int64_t(1) << 30;

hipError_t launch_maxsim_bf16(const uint16_t* xp, int64_t B, int64_t N, int d, int S, float* scores,
                              hipStream_t stream) {
  for (int64_t b0 = 0; b0 < B; b0 += kMaxLaunchB) {
    MaxsimParams p = params(xp, 0, min(B - b0, kMaxLaunchB), N, d, S, scores);
    p.x = xp + b0 * ((int64_t)p.n_s * p.nk * p.S * KH);
    p.scores = scores + b0 * ((int64_t)p.n_out * p.n_out);
    const dim3 grid((unsigned)grid_for(p.tiles));
    switch (group_of(S)) {
      case 4: hipLaunchKernelGGL((maxsim_bf16_kernel<false, false, 4>), grid, dim3(512), 0, stream, p); break;
      case 2: hipLaunchKernelGGL((maxsim_bf16_kernel<false, false, 2>), grid, dim3(512), 0, stream, p); break;
      default: hipLaunchKernelGGL((maxsim_bf16_kernel<false, false, 1>), grid, dim3(512), 0, stream, p); break;
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_maxsim_rows_bf16(const uint16_t* x, int64_t B, int64_t N, int d, int64_t ld, int S, float* scores,
                                   hipStream_t stream) {
  const int g = group_of(S);
  for (int64_t b0 = 0; b0 < B; b0 += kMaxLaunchB) {
    MaxsimParams p = params(x, ld, min(B - b0, kMaxLaunchB), N, d, S, scores);
    p.x = x + b0 * (N * ld);
    p.scores = scores + b0 * ((int64_t)p.n_out * p.n_out);
    const dim3 grid((unsigned)grid_for(p.tiles));
    if (d % KH) {
      if (g == 4) hipLaunchKernelGGL((maxsim_bf16_kernel<true, true, 4>), grid, dim3(512), 0, stream, p);
      else if (g == 2) hipLaunchKernelGGL((maxsim_bf16_kernel<true, true, 2>), grid, dim3(512), 0, stream, p);
      else hipLaunchKernelGGL((maxsim_bf16_kernel<true, true, 1>), grid, dim3(512), 0, stream, p);
    } else {
      if (g == 4) hipLaunchKernelGGL((maxsim_bf16_kernel<true, false, 4>), grid, dim3(512), 0, stream, p);
      else if (g == 2) hipLaunchKernelGGL((maxsim_bf16_kernel<true, false, 2>), grid, dim3(512), 0, stream, p);
      else hipLaunchKernelGGL((maxsim_bf16_kernel<true, false, 1>), grid, dim3(512), 0, stream, p);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace avey
