// LDS tiles filled by direct global->LDS loads (global_load_lds_dwordx4).
//
// A tile holds ROWS rows of CH 16-byte chunks (CH = 4, 8 or 16), stored
// densely (row stride CH*16 bytes) with an XOR swizzle: logical chunk c of
// row r sits at physical chunk c ^ sw(r), with x = (r / RP) % CH (RP = 16/CH
// rows share one 256-byte line of the 64 LDS banks) and sw(r) = x rotated
// left by one bit within log2(CH) bits.  Two read patterns are then
// bank-conflict free:
//  * 16 bytes per lane, one row per lane (16 consecutive rows, one chunk):
//    sw is a bijection of x;
//  * the transposing read (below), where 16 lanes fetch 4 consecutive rows
//    x 32 bytes (chunks c, c+1 with c even): rotating makes sw of the two
//    row pairs differ in a bit above bit 0, so the 8 chunks land apart.
//
// A direct load writes a wave's 64 lanes to 64 consecutive 16-byte LDS
// slots (base + lane*16): load i of a tile fills rows i*64/CH ... and lane l
// fetches row i*64/CH + l/CH, logical chunk (l % CH) ^ sw(row); since
// x = (4i + l/16) % CH and rotation is linear over XOR, that chunk is
// (l % CH) ^ rot(l/16) ^ rot(4i % CH).  The loads complete asynchronously:
// wait_async() (vmcnt 0) and a workgroup barrier publish the tile.
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

    __device__ static constexpr int rot(int x) {   // rotate left by 1 within log2(CH) bits
        return ((x << 1) & (CH - 1)) | (x >> (CH == 16 ? 3 : CH == 8 ? 2 : 1));
    }
    __device__ static constexpr int swz(int r) { return rot((r / RP) & (CH - 1)); }
    // byte offset of logical chunk c of row r
    __device__ static constexpr int off(int r, int c) { return r * kStride + ((c ^ swz(r)) << 4); }
};

// Issue this wave's share of the loads of one tile whose row r is at
// base + r * row_stride bytes.  Rows at or past `valid_rows` are read from
// row valid_rows - 1 instead (the caller makes such rows harmless).
template <int ROWS, int CH, int NWAVES>
__device__ __forceinline__ void stage_rows_async(char *tile, int wave, int lane, const void *base,
                                                 size_t row_stride, int valid_rows) {
    using T = SwzTile<ROWS, CH>;
    lds_byte *lds = (lds_byte *)tile;   // the tile lives in __shared__ memory
    const char *src = (const char *)base;
    const int a = (lane & (CH - 1)) ^ T::rot((lane >> 4) & (CH - 1));
    for (int i = wave; i < T::kInstr; i += NWAVES) {
        int r = i * (64 / CH) + lane / CH;
        r = r < valid_rows ? r : valid_rows - 1;
        const int c = a ^ T::rot((4 * i) & (CH - 1));
        __builtin_amdgcn_global_load_lds((const void *)(src + (size_t)r * row_stride + c * 16),
                                         lds + i * 1024, 16, 0, 0);
    }
}

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
