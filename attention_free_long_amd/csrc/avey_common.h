// Device helpers shared by the gfx950 kernels of libavey.
//
// Operand tiles live in LDS as [rows][64] bf16 (128-byte rows). The sixteen-byte chunk c of
// row r is stored at chunk position c ^ swz(r), with one of two swizzles:
//   * SWZ_ROW  swz(r) = (r >> 1) & 7        for tiles filled by direct global -> LDS copies
//     (one copy instruction writes 8 whole rows);
//   * SWZ_DIAG swz(r) = (r ^ (r >> 3)) & 7  for tiles written by register transposes (one
//     write instruction covers rows 8 apart).
// The LDS has 64 four-byte banks and serves a 16-byte-per-lane access for 16 lanes per cycle, so
// an MFMA fragment read (16 consecutive rows, one chunk each) must hit 16 distinct 16-byte slots
// of a 256-byte window: rows 2m and 2m+1 differ by 128 bytes, and the swizzle spreads the eight
// row pairs over the eight chunk positions. Both
// keep the fragment address of row block mb (32 rows) a fixed offset from block 0 (SWZ_DIAG
// also swaps k-steps 0<->2 and 1<->3 on odd blocks), so a wave needs only 4 address registers
// per operand.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace avey {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int KC = 64;              // K elements per staged chunk (one 128-byte LDS row)
constexpr int ROWB = 128;           // bytes per LDS row
constexpr int NXCD = 8;             // XCDs of an MI355X; workgroups are dealt round-robin

enum Swizzle { SWZ_ROW = 0, SWZ_DIAG = 1 };

template <Swizzle W>
__device__ __forceinline__ uint32_t swz(int r) {
  return W == SWZ_ROW ? (uint32_t)((r >> 1) & 7) : (uint32_t)((r ^ (r >> 3)) & 7);
}

// Byte offset of logical 16-byte chunk c of row r.
template <Swizzle W>
__device__ __forceinline__ uint32_t lds_off(int r, int c) {
  return (uint32_t)r * ROWB + (((uint32_t)c ^ swz<W>(r)) << 4);
}

// Per-lane fragment offsets for the four k-steps of a chunk, row block starting at r0 (a
// multiple of 64). Block mb of 32 rows is at frag[ks'] + mb * 32 * ROWB with ks' = ks for
// SWZ_ROW and ks' = ks ^ (2 * (mb & 1)) for SWZ_DIAG.
template <Swizzle W>
__device__ __forceinline__ void frag_offsets(uint32_t (&frag)[4], int r0, int lane) {
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) frag[ks] = lds_off<W>(r0 + (lane & 31), 2 * ks + (lane >> 5));
}

template <Swizzle W>
__device__ __forceinline__ constexpr int frag_ks(int ks, int mb) {
  return W == SWZ_ROW ? ks : (ks ^ (2 * (mb & 1)));
}

__device__ __forceinline__ uint4 lds_read16(const uint8_t* base, uint32_t off) {
  return *reinterpret_cast<const uint4*>(base + off);
}

__device__ __forceinline__ void lds_write16(uint8_t* base, uint32_t off, uint4 v) {
  *reinterpret_cast<uint4*>(base + off) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// 32x32x16 bf16 MFMA: acc[i][j] += sum_k A[i][k] B[k][j]. Lane l supplies A row (l & 31) and
// B column (l & 31), k = 8 * (l >> 5) + 0..7. Result element v of lane l is
// row 8 * (v >> 2) + 4 * (l >> 5) + (v & 3), column l & 31.
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int v, int lane) { return ((v >> 2) << 3) + ((lane >> 5) << 2) + (v & 3); }

// Sum of squares of eight bf16 values, accumulated in fp32.
__device__ __forceinline__ float sumsq8(uint4 v, float acc) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, v.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, v.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, v.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, v.w), acc, false);
  return acc;
}

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Pack 16-bit half `h` (0 low, 1 high) of a and of b as (a_h, b_h).
__device__ __forceinline__ uint32_t pick16(uint32_t a, uint32_t b, int h) {
  return h ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

// Raw buffer descriptor over [base, base + bytes). Loads at offsets >= bytes return zero.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// The same over a base address the compiler cannot prove wave-uniform (one computed from
// values that went through the vector unit): the address and size are read from the first
// lane, so the descriptor lives in scalar registers. A descriptor the compiler takes as per-lane
// turns every load through it into a loop over its distinct values.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  const uint64_t addr = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)addr);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(addr >> 32));
  return make_rsrc(reinterpret_cast<const void*>(((uint64_t)hi << 32) | lo),
                   __builtin_amdgcn_readfirstlane(bytes));
}

// An offset past every descriptor this library builds (all are < 2^31 bytes): reads as zero.
constexpr uint32_t OOB = 0x80000000u;

// 16-byte load through a buffer descriptor (voff + soff bytes from the base).
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}

// 16-byte store through a buffer descriptor. A lane whose offset is out of range (OOB) writes
// nothing, so a wave can issue the same number of stores whatever its lanes' validity. On this
// GPU one vector-memory counter (vmcnt) counts buffer loads, direct-to-LDS copies and buffer
// stores together, and a wave's vector-memory operations report completion in the order they
// were issued. A wait for "at most n outstanding" therefore completes exactly the operations
// issued before the last n, and the pipelined kernels add the stores they issued after a chunk's
// copies to n when they wait for that chunk. kPolicy is the cache-policy operand (2 sets the
// non-temporal bit).
template <int kPolicy = 0>
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint4 v) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, soff, kPolicy);
}

// Direct global -> LDS copy of 16 bytes per lane: lane l writes lds_base + 16 * l, where
// lds_base must be the same for the whole wave.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t* lds_base, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds_base, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier for LDS traffic only. __syncthreads() also drains every outstanding global
// load, including direct-to-LDS copies of a stage that is not read yet; this one waits for the
// wave's own LDS operations and leaves global loads in flight. The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Barrier after which every wave's direct-to-LDS copies (and LDS writes) are complete.
__device__ __forceinline__ void copy_sync() {
  asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Workgroup id -> logical tile so that each XCD works through one contiguous range of
// logical tiles (workgroups are dealt to the XCDs round-robin by id).
__device__ __forceinline__ int64_t xcd_remap(int64_t wg, int64_t total) {
  const int64_t x = wg % NXCD, l = wg / NXCD;
  const int64_t q = total / NXCD, r = total % NXCD;
  return x * q + (x < r ? x : r) + l;
}

// Compile-time loop: f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}).
template <int I, int N, class F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }

}  // namespace avey
