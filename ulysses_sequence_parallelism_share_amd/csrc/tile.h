// LDS tiles filled by direct global->LDS loads (global_load_lds_dwordx4).
//
// A tile holds ROWS rows of CH 16-byte chunks (CH = 4, 8 or 16), stored
// densely (row stride CH*16 bytes) with an XOR swizzle: logical chunk c of
// row r sits at physical chunk c ^ sw(r), sw(r) = (r / RP) & (CH - 1), where
// RP = 16 / CH rows share one 256-byte line of the 64 LDS banks.  Sixteen
// consecutive rows read at one logical chunk then touch 16 distinct 16-byte
// bank groups, so the 16-bytes-per-lane MFMA operand reads (one row per
// lane) are conflict-free.
//
// A direct load writes a wave's 64 lanes to 64 consecutive 16-byte LDS
// slots (base + lane*16): load i of a tile fills rows i*64/CH ... and lane l
// fetches row i*64/CH + l/CH, logical chunk (l % CH) ^ sw(row), which for
// every CH reduces to (l % CH) ^ ((4i + l/16) % CH).  The loads complete
// asynchronously: wait_async() (vmcnt 0) and a workgroup barrier publish
// the tile.
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

    __device__ static constexpr int swz(int r) { return (r / RP) & (CH - 1); }
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
    const int a = lane & (CH - 1), b = lane >> 4;
    for (int i = wave; i < T::kInstr; i += NWAVES) {
        int r = i * (64 / CH) + lane / CH;
        r = r < valid_rows ? r : valid_rows - 1;
        const int c = a ^ ((4 * i + b) & (CH - 1));
        __builtin_amdgcn_global_load_lds((const void *)(src + (size_t)r * row_stride + c * 16),
                                         lds + i * 1024, 16, 0, 0);
    }
}

// Wait for this wave's outstanding direct loads (vmcnt = 0).
__device__ __forceinline__ void wait_async() { __builtin_amdgcn_s_waitcnt(0x0F70); }
