// LDS tiles filled by direct global->LDS loads (global_load_lds_dwordx4).
//
// A tile holds ROWS rows of CH 16-byte chunks (CH = 4, 8 or 16), stored
// densely (row stride CH*16 bytes) with an XOR swizzle: logical chunk c of
// row r sits at physical chunk c ^ sw(r).  RP = 16/CH rows share one
// 256-byte line of the 64 LDS banks (16 chunk slots).  Two read patterns
// must be bank-conflict free:
//  * 16 bytes per lane, one row per lane, 16 consecutive rows at one chunk
//    (served 16 lanes at a time): (r % RP, sw(r)) must be distinct over the
//    16 rows, i.e. sw a bijection of x = (r / RP) % CH;
//  * the transposing read (below), served 32 lanes at a time: 4 consecutive
//    rows r0..r0+3 (r0 % 4 == 0) x 64 bytes (chunks c..c+3, c % 4 == 0)
//    must fill 16 distinct chunk slots, so the sw of rows sharing a line
//    slot must differ in bit 2 or 3.
// CH = 16: sw swaps the two 2-bit halves of x = r % 16 (rows r0+z get
// 4z + const); CH = 8: x = (r/2) % 8, sw = (x % 2) * 4 + x / 2 (rows r0,
// r0+1 and r0+2, r0+3 differ in bit 2); CH = 4: sw = x.
//
// A direct load writes a wave's 64 lanes to 64 consecutive 16-byte LDS
// slots (base + lane*16): load i of a tile fills rows i*64/CH ... and lane l
// fetches row i*64/CH + l/CH, logical chunk (l % CH) ^ sw(row).  The loads
// complete asynchronously: wait_async() (vmcnt 0) and a workgroup barrier
// publish the tile.
#pragma once

#include "common.h"

typedef __attribute__((address_space(3))) char lds_byte;

template <int ROWS, int CH>
struct SwzTile {
    static_assert(CH == 4 || CH == 8 || CH == 16, "chunks per row");
    static constexpr int RP = 16 / CH;
    static constexpr int kStride = CH * 16;
    static constexpr int kBytes = ROWS * CH * 16;
    static constexpr int kInstr = ROWS * CH / 64;
    static_assert(kInstr * 64 == ROWS * CH, "tile must be whole wave-wide loads");

    __device__ static constexpr int swz(int r) {
        const int x = (r / RP) & (CH - 1);
        return CH == 16 ? (((x & 3) << 2) | (x >> 2)) : CH == 8 ? (((x & 1) << 2) | (x >> 1)) : x;
    }
    // byte offset of logical chunk c of row r
    __device__ static constexpr int off(int r, int c) { return r * kStride + ((c ^ swz(r)) << 4); }
};

// Issue this wave's share of the direct loads of one tile.  Source row r of
// the tile (relative to the tile's base address) lies at byte offset
//     (r >> gshift) * tok_bytes + (r & (2^gshift - 1)) * row_bytes,
// which covers rows with one constant stride (gshift = 0, tok_bytes = the
// stride) and the rows of several heads of one token taken together (2^gshift
// heads per token, row_bytes apart, tokens tok_bytes apart).  The per-lane
// part of every load's address is computed once (init); staging a full tile
// then costs one address add per load.  In a tile with fewer than ROWS valid
// rows (the last one), rows at or past `valid_rows` are read from row
// valid_rows - 1 instead (the caller makes such rows harmless).
// One direct global->LDS load of 16 bytes per lane (lane i to lds + 16 i:
// the LDS base goes in M0), issued through inline assembly.  The compiler's
// own form makes every later transposing LDS read wait for all direct loads
// in flight (it cannot tell that they write other bytes), which drains the
// prefetch of the next tile; here the callers' s_waitcnt vmcnt and
// workgroup barrier alone publish the data (the compiler's waits for its
// own loads stay correct: loads complete in issue order).  M0 is written
// inside the statement and listed as clobbered; the compiler emits no M0
// access of its own in these kernels (checked in their assembly).  Passing
// M0 as an input operand instead ("{m0}") yields the same instructions in a
// slightly different order, runs at the same speed, and measured 2.3x the
// L2-miss fetch of the dK/dV kernel (FETCH_SIZE), so this form is kept.
__device__ __forceinline__ void dma16(const void *g, lds_byte *l) {
    const uint32_t la = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(la) : "memory", "m0");
}

// The same load with a wave-uniform 64-bit base in SGPRs and a 32-bit
// per-lane byte offset (the saddr form): no per-lane 64-bit address adds.
__device__ __forceinline__ void dma16s(const void *sbase, uint32_t voff, lds_byte *l) {
    const uint32_t la = (uint32_t)(uintptr_t)l;
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(voff), "s"(sbase), "s"(la) : "memory", "m0");
}

// SADDR selects the saddr form (the tile base must be wave-uniform, and the
// tile must span less than 4 GiB); with it the forward, dQ and cross-entropy
// GEMM kernels measured 0.7-3 % faster, the dK/dV kernel 1 % slower, so that
// one keeps 64-bit per-lane addresses.
template <int ROWS, int CH, int NWAVES, bool SADDR = true>
struct RowStager {
    using T = SwzTile<ROWS, CH>;
    static constexpr int kPer = (T::kInstr + NWAVES - 1) / NWAVES;   // loads per wave, at most
    uint32_t off[kPer];
    uint32_t tok_bytes, row_bytes;
    int gshift;

    __device__ uint32_t row_off(int r) const {
        return (uint32_t)(r >> gshift) * tok_bytes + (uint32_t)(r & ((1 << gshift) - 1)) * row_bytes;
    }
    __device__ static bool mine(int wave, int k) {
        return T::kInstr % NWAVES == 0 || wave + k * NWAVES < T::kInstr;
    }
    __device__ void init(int wave, int lane, uint32_t tok_bytes_, uint32_t row_bytes_, int gshift_) {
        tok_bytes = tok_bytes_;
        row_bytes = row_bytes_;
        gshift = gshift_;
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
            const int i = mine(wave, k) ? wave + k * NWAVES : 0;
            const int rs = i * (64 / CH) + lane / CH;
            off[k] = row_off(rs) + (uint32_t)(((lane & (CH - 1)) ^ T::swz(rs)) << 4);
        }
    }
    __device__ void issue(char *tile, int wave, int lane, const void *base, int valid_rows) const {
        lds_byte *lds = (lds_byte *)tile;
        const char *src = (const char *)base;
        if (valid_rows >= ROWS) {
#pragma unroll
            for (int k = 0; k < kPer; ++k)
                if (mine(wave, k)) {
                    if constexpr (SADDR)
                        dma16s(src, off[k], lds + (wave + k * NWAVES) * 1024);
                    else
                        dma16((const void *)(src + off[k]), lds + (wave + k * NWAVES) * 1024);
                }
            return;
        }
        for (int k = 0; k < kPer; ++k) {
            if (!mine(wave, k)) continue;
            const int i = wave + k * NWAVES;
            const int rs = i * (64 / CH) + lane / CH;          // LDS row of this slot
            const int r = rs < valid_rows ? rs : valid_rows - 1; // source row it holds
            const int c = (lane & (CH - 1)) ^ T::swz(rs);
            if constexpr (SADDR)
                dma16s(src, row_off(r) + (uint32_t)(c * 16), lds + i * 1024);
            else
                dma16((const void *)(src + row_off(r) + c * 16), lds + i * 1024);
        }
    }
};

// Wait for this wave's outstanding direct loads (vmcnt = 0).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// ---------------------------------------------------------------------------
// Transposing operand read (ds_read_b64_tr_b16).
//
// Within each group of 16 lanes, lane i of the read receives as its element k
// (k = 0..3) the element i % 4 of the 4 consecutive 16-bit values addressed
// by lane 4k + i/4 of the group.
//
// read_tr8 builds, from a tile T stored as [k-row][m] (m contiguous), the
// MFMA operand in which lane l supplies index m0 + l % 32 and, for half
// h = l / 32, the k-rows kbase + 4h + {0,1,2,3} (elements 0..3) and
// kbase + 8 + 4h + {0,1,2,3} (elements 4..7) -- the rows that accumulator
// registers 8s..8s+7 of a 32x32 block hold for lane half h.  kbase must be a
// multiple of 16.  Group G = l / 16 covers m0 + 16 (G % 2) ... + 15; its
// lane j fetches row kbase + 4h + j/4 (+ 8), columns m + 4 (j % 4) .. +3.
// ---------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <class T>
__device__ __forceinline__ bf16x8 read_tr8(const char *tile, int kbase, int m0, int lane) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int G = lane >> 4, j = lane & 15;
    const int m = m0 + 16 * (G & 1) + 4 * (j & 3);
    const int row = kbase + 4 * (G >> 1) + (j >> 2);
    const int c = m >> 3, sub = (m & 7) * 2;
    const char *p0 = tile + T::off(row, c) + sub;
    const char *p1 = tile + T::off(row + 8, c) + sub;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p0);
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, v);
}

// The same operand with contiguous k-rows per lane: lane l supplies index
// m0 + l % 32 and k-rows kbase + 8h + {0..7} (h = l / 32), the k-slots a
// 16-byte read of a k-contiguous tile gives (chunk 2s + h of k16-step s), so
// the two kinds of operand can be multiplied together.  Each 32-lane half
// still reads 4 consecutive rows at a time (rows kbase + 8h + j/4, then
// + 4), which keeps the swizzle's conflict-free pattern.
template <class T>
__device__ __forceinline__ bf16x8 read_tr8k(const char *tile, int kbase, int m0, int lane) {
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int G = lane >> 4, j = lane & 15;
    const int m = m0 + 16 * (G & 1) + 4 * (j & 3);
    const int row = kbase + 8 * (G >> 1) + (j >> 2);
    const int c = m >> 3, sub = (m & 7) * 2;
    const char *p0 = tile + T::off(row, c) + sub;
    const char *p1 = tile + T::off(row + 4, c) + sub;
    const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p0);
    const s16x4 y = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(lds_byte *)p1);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
    return __builtin_bit_cast(bf16x8, v);
}
