// Small device helpers shared by the bf16 attention kernels (forward and
// backward): vector types, the 16x16x32 bf16 MFMA, direct-to-LDS buffer loads,
// buffer resources, and (for the backward's tiles) LDS addressing with a
// row-dependent chunk swizzle and the transposing LDS read.  Internal header.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace txl {
namespace tiles {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define TXL_LDS_AS __attribute__((address_space(3)))

constexpr int DH = 64;             // head width of these kernels
constexpr int CPR = DH / 8;        // 16-byte chunks per 64-element bf16 row
constexpr float LN2 = 0.69314718055994530942f;
constexpr float LOG2E = 1.44269504088896340736f;

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Chunk swizzle of an LDS tile of 64-element bf16 rows: chunk c of row r sits
// at position c ^ swz(r).  Measured with the LDS bank-conflict counter on
// gfx950, both access patterns used on these tiles run without conflicts: a
// 16-row fragment read (one 16-byte chunk per lane) and a transposing read
// (8 bytes per lane from rows 4 g .. 4 g + 3); with the pattern (r >> 1) & 7
// instead, the transposing reads take two passes.
__device__ __forceinline__ int swz(int r) { return r & (CPR - 1); }

// Orders this wave's LDS accesses for the compiler without waiting.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(TXL_LDS_AS const void *)p;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, 0x00020000);
}

// Direct HBM -> LDS load of 16 bytes per lane: lane l writes LDS byte address
// lds + 16 l (lds is wave-uniform).  Offsets at or past the resource size read
// zeros.  Inline assembly, so the compiler does not track it: the caller waits
// (s_waitcnt vmcnt(0), then a barrier) before anything reads the target.
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds)
{
    uint32_t saved;
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(rsrc), "s"(lds)
        : "memory");
}

// 16-byte global load through a buffer resource (zeros past its size).
__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t rsrc, uint32_t off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
}

// Row fragment of an LDS tile (64-element bf16 rows, swizzled): the 8
// elements 32 kk + 8 g .. + 7 of row `row` (A or B operand of a 16x16x32
// MFMA whose contraction runs over the row).
__device__ __forceinline__ bf16x8 row_frag(const u32x4 *tile, int row, int kk, int g)
{
    return __builtin_bit_cast(bf16x8, tile[row * CPR + ((4 * kk + g) ^ swz(row))]);
}

// Column fragment through the transposing LDS read: for lane (g, n) the
// elements [rows rb + 4 g + e][col 16 dt + n] (e = 0..3, k-slots 0..3) and
// [rows rb + 16 + 4 g + e][same col] (k-slots 4..7).  This is the operand
// layout of a 16x16x32 MFMA whose contraction runs over 32 tile rows taken
// in the order {4g..4g+3, 16+4g..16+4g+3} per lane group; a C-layout result
// of two 16-row MFMA tiles packs into the matching B/A operand without data
// movement.  rb must be a multiple of 4.
__device__ __forceinline__ bf16x8 col_frag(const u32x4 *tile, int rb, int dt, int g, int n)
{
    TXL_LDS_AS char *base = (TXL_LDS_AS char *)(TXL_LDS_AS void *)tile;
    const int chunk = 2 * dt + ((n >> 1) & 1);
    const int r0 = rb + 4 * g + (n >> 2), r1 = r0 + 16;
    const int off0 = (r0 * CPR + (chunk ^ swz(r0))) * 16 + 8 * (n & 1);
    const int off1 = (r1 * CPR + (chunk ^ swz(r1))) * 16 + 8 * (n & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(base + off0));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(base + off1));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}

// Half of col_frag: rows rb + 4 g + e only (k-slots 0..3); k-slots 4..7 zero.
__device__ __forceinline__ bf16x8 col_frag_lo(const u32x4 *tile, int rb, int dt, int g, int n)
{
    TXL_LDS_AS char *base = (TXL_LDS_AS char *)(TXL_LDS_AS void *)tile;
    const int chunk = 2 * dt + ((n >> 1) & 1);
    const int r0 = rb + 4 * g + (n >> 2);
    const int off0 = (r0 * CPR + (chunk ^ swz(r0))) * 16 + 8 * (n & 1);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(base + off0));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], 0u, 0u});
}

// The same reads with the lane part of the address computed once.  For a
// block of rows starting at a multiple of 16, swz(row) depends on the lane
// only: (16 k + 4 g + (n >> 2)) & 7 = (4 g + (n >> 2)) & 7.
//   row_lane_off: byte offset of lane (g, n)'s chunk (4 kk + g) in row n of
//     the block -- row fragments;
//   tr_lane_off: byte offset of lane (g, n)'s 8 bytes for output column
//     block dt in rows 4 g + (n >> 2) of the block -- transposing reads.
__device__ __forceinline__ int row_lane_off(int kk, int g, int n)
{
    return (n * CPR + ((4 * kk + g) ^ swz(n))) * 16;
}
__device__ __forceinline__ int tr_lane_off(int dt, int g, int n)
{
    const int r = 4 * g + (n >> 2);
    return (r * CPR + ((2 * dt + ((n >> 1) & 1)) ^ swz(r))) * 16 + 8 * (n & 1);
}
// Row fragment of the 16-row block at byte `blk` (row16 * CPR * 16 bytes into
// a tile, row16 a multiple of 16) with a precomputed row_lane_off.
__device__ __forceinline__ bf16x8 row_frag_at(const TXL_LDS_AS char *blk, int lane_off)
{
    return *(const TXL_LDS_AS bf16x8 *)(blk + lane_off);
}
// col_frag over the 32 rows starting at byte `blk` (a 16-row-aligned block)
// with a precomputed tr_lane_off; hi = false leaves k-slots 4..7 zero.
__device__ __forceinline__ bf16x8 col_frag_at(const TXL_LDS_AS char *blk, int lane_off, bool hi = true)
{
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(blk + lane_off));
    const u32x2 l2 = __builtin_bit_cast(u32x2, lo);
    u32x2 h2 = {0u, 0u};
    if (hi) h2 = __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                     (TXL_LDS_AS i16x4 *)(blk + 16 * CPR * 16 + lane_off)));
    return __builtin_bit_cast(bf16x8, u32x4{l2[0], l2[1], h2[0], h2[1]});
}
// One half of col_frag_at (rows 4 g + e of the block at `blk`), as 2 dwords.
__device__ __forceinline__ u32x2 tr_half(const TXL_LDS_AS char *blk, int lane_off)
{
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((TXL_LDS_AS i16x4 *)(blk + lane_off)));
}
__device__ __forceinline__ const TXL_LDS_AS char *lds_bytes(const u32x4 *tile)
{
    return (const TXL_LDS_AS char *)(const TXL_LDS_AS void *)tile;
}

// Four floats to consecutive LDS words (4-byte aligned only).  The compiler
// pairs them into two-word stores (ds_write2_b32, half the store instructions);
// in the current forward kernel that measured 3.5% faster than four one-word
// stores (37.1 vs 38.4 us at B8 H16 L512 M512) and freed the registers its
// unmasked instance had spilled.  (An earlier build of the kernel measured the
// opposite, ~10% slower.)
__device__ __forceinline__ void lds_store4(float *dst, f32x4 v)
{
    TXL_LDS_AS float *p = (TXL_LDS_AS float *)dst;
    p[0] = v[0];
    p[1] = v[1];
    p[2] = v[2];
    p[3] = v[3];
}

// Two C-layout MFMA results (4 rows each per lane) as one 8-slot bf16 operand.
__device__ __forceinline__ bf16x8 pack8(f32x4 a, f32x4 b)
{
    const f32x8 x = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    return __builtin_convertvector(x, bf16x8);
}

}  // namespace tiles
}  // namespace txl
