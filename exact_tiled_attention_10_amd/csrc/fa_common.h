// Shared device helpers for the gfx950 attention kernels.
//
// MFMA layout facts used throughout (CDNA3/CDNA4 matrix-core operand layout,
// 64-lane wavefront):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row m = l % 32 and 8 k-values chosen by (l / 32, t)
//     B: lane l holds column n = l % 32 and the same 8 k-values
//     D: lane l, register r holds D[8*(r/4) + 4*(l/32) + r%4][l % 32]
//   v_mfma_f32_32x32x2_f32: as above with one k-value per lane, k = l / 32.
// The mapping of (l / 32, t) to k never matters to the kernels: A and B always
// carry the same logical key (or feature) in the same slot, and the product
// sums over every slot.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma_32x32x16_bf16(const bf16x8& a,
                                                     const bf16x8& b,
                                                     const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma_32x32x2_f32(float a, float b,
                                                   const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Round-to-nearest-even float -> bf16 pair packed in one dword (lo = a); one
// v_cvt_pk_bf16_f32 (two scalar conversions would cost a shift and an or more).
// The value unchanged, but unknown to the compiler from here on: per-lane
// offsets derived from it inside a loop are formed where they are used
// instead of being computed once before the loop and held in registers for
// its whole length (kernels whose registers are taken by operands and
// accumulators have no room for them).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Low (sel = 0x05040100) or high (sel = 0x07060302) 16-bit halves of a and b
// packed as {a_half, b_half}.
__device__ __forceinline__ uint32_t pack_lo16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi16(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}

__device__ __forceinline__ float wave_xor32(float x) {
  // exchange with the lane 32 positions away (the other half of the wave)
  return __shfl_xor(x, 32, 64);
}

// Position of a 4-row group inside its 16-row chunk in a transposed operand
// tile (V^T in the forward, Q^T and dO^T in the backward).  A 32x32 MFMA
// accumulator gives lane half h rows {4h..4h+3, 8+4h..8+4h+3} of each 16-row
// chunk in registers t = 0..7; storing the groups in the order 0, 2, 1, 3 puts
// exactly those 8 rows at positions 8h..8h+7, so the matching A operand is one
// 16-byte LDS read.
__device__ __forceinline__ int tr_group_pos(int lg) { return ((lg & 1) << 1) | (lg >> 1); }

// ---------------------------------------------------------------------------
// LDS tiles filled by direct global->LDS DMA.
//
// global_load_lds_dwordx4 writes lane i's 16 bytes to LDS base + 16*i, so a
// wave instruction fills 1 KiB contiguously and rows cannot be padded.  Bank
// conflicts are avoided with an XOR swizzle instead: inside row r of a tile
// with CPR 16-byte chunks per row, chunk c is stored at position c ^ swz(r).
//
// gfx950's LDS serves 256 bytes (64 banks x 4 B) per cycle: 16 lanes of a
// ds_read_b128, 32 lanes of a ds_read_b64_tr_b16.  A conflict-free access
// therefore touches 16 distinct 16-byte slots modulo 256 bytes.  Two swizzles
// cover the two read patterns the kernels use:
//   SWZ_ROWS  16 consecutive rows read at the same chunk (a row-operand
//             read: lane n reads row n).  CPR 16 and 32: swz = r % 16;
//             CPR 8 (two rows per 256 B): swz = (r / 2) % 8.
//   SWZ_TR    transposing reads: rows r0..r0+3 (r0 % 4 == 0) at four
//             consecutive chunks 4b..4b+3.  CPR 16 and 32: swz = 4 (r % 4);
//             CPR 8: swz = 4 ((r / 2) % 2).
//   SWZ_BOTH  both patterns on one tile: CPR 16 and 32: swz = 4 (r % 4) +
//             (r / 4) % 4; CPR 8: swz = 4 ((r / 2) % 2) + (r / 4) % 4.
// (A row of CPR 32 spans 512 bytes, so rows are 256-byte aligned like CPR 16
// and the same swizzles apply.)
// ---------------------------------------------------------------------------
enum { SWZ_ROWS = 0, SWZ_TR = 1, SWZ_BOTH = 2 };

template <int CPR, int KIND>
__device__ __forceinline__ int swz(int r) {
  static_assert(CPR == 8 || CPR == 16 || CPR == 32, "rows of 64, 128 or 256 bf16");
  if (KIND == SWZ_ROWS) return CPR >= 16 ? (r & 15) : ((r >> 1) & 7);
  if (KIND == SWZ_TR) return CPR >= 16 ? ((r & 3) << 2) : (((r >> 1) & 1) << 2);
  return CPR >= 16 ? (((r & 3) << 2) | ((r >> 2) & 3)) : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Byte offset of element column `col` (a multiple of 4) of row `row`.
template <int CPR, int KIND>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * CPR * 16 + (((col >> 3) ^ swz<CPR, KIND>(row)) << 4) + ((col & 7) << 1);
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(lds_void*)p;
}

// One 16-byte global -> LDS DMA per lane: global address gbase + voff (gbase
// wave-uniform), LDS address lds + 16 * lane (lds wave-uniform).
//
// Issued as inline assembly on purpose: through the compiler builtin, the
// waitcnt pass cannot tell that a DMA into one LDS stage does not alias reads
// of the other stage, and waits for the in-flight prefetch before every LDS
// read.  Here completion is the caller's job: wait_vmem() and a workgroup
// barrier before any wave reads the stage.
__device__ __forceinline__ void dma16(const void* gbase, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(gbase), "s"(lds)
               : "memory", "m0");
}

// One 16-byte global -> LDS DMA per lane through a buffer resource: lane i
// reads rsrc.base + voff (0 when voff is past the resource's byte count) and
// writes LDS lds + 16 i.  Inline assembly for the reason given at dma16.
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, unsigned voff, unsigned lds) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(lds)
               : "memory", "m0");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each 16-lane group, the
// lane 4j + c reads 4 bf16 of "row" j; output lane 4c + e receives element e
// of rows j = 0..3.  So if lane 4j + c points at row (r0 + j), columns
// (n0 + 4c .. n0 + 4c + 3), output lane i holds column n0 + i of rows
// r0 .. r0 + 3: a k-contiguous MFMA operand read from an n-contiguous tile.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* lds_ptr) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)lds_ptr));
}

// Wait until all of this wave's vector memory operations (including LDS DMA)
// have completed.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Wait until at most N of this wave's vector memory operations are still
// outstanding (they complete in issue order): N = the DMAs of the tiles that
// may stay in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_but() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Work-tile order for the forward and backward grids.
//
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i lands on
// XCD i % 8), and each XCD has its own L2.  When the (batch*head) count
// divides by 8, every XCD is given whole heads, so the key/value tiles a head
// streams stay in one L2; within an XCD the tiles are issued heaviest first
// (highest query tile first, which under causal masking carries the most key
// tiles) so the long tiles do not trail at the end.  Otherwise fall back to
// heaviest first across all heads.
__device__ __forceinline__ void map_tile(int bid, int BH, int ntiles, bool heavy_first,
                                         int* bh, int* tile) {
  int t, h;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7;
    const int j = bid >> 3;
    const int hpx = BH >> 3;
    t = j / hpx;
    h = xcd * hpx + (j - t * hpx);
  } else {
    t = bid / BH;
    h = bid - t * BH;
  }
  *bh = h;
  *tile = heavy_first ? (ntiles - 1 - t) : t;
}

// map_tile for kernels of which several workgroups share a CU from the
// start: consecutive passes of `pass` workgroups per XCD (one per compute
// unit) run in alternating directions, so the compute unit that takes the
// heaviest tile of one pass takes the lightest of the next and every unit's
// total comes out alike.
__device__ __forceinline__ void map_tile_snake(int bid, int BH, int ntiles, bool heavy_first,
                                               int pass, int* bh, int* tile) {
  int t, h;
  if ((BH & 7) == 0) {
    const int xcd = bid & 7;
    int j = bid >> 3;
    const int hpx = BH >> 3;
    const int nx = hpx * ntiles;
    const int p = j / pass;
    if (p & 1) {
      const int len = min(pass, nx - p * pass);
      j = p * pass + (len - 1 - (j - p * pass));
    }
    t = j / hpx;
    h = xcd * hpx + (j - t * hpx);
  } else {
    int j = bid;
    const int n = BH * ntiles;
    const int p = j / (8 * pass);
    if (p & 1) {
      const int len = min(8 * pass, n - p * 8 * pass);
      j = p * 8 * pass + (len - 1 - (j - p * 8 * pass));
    }
    t = j / BH;
    h = j - t * BH;
  }
  *bh = h;
  *tile = heavy_first ? (ntiles - 1 - t) : t;
}

}  // namespace fa
