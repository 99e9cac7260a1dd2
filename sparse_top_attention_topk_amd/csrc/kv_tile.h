// The gathered KV tile in LDS: BLK top-k slots x d_qk bf16, one row per slot.
//
// The tile is filled from the token's index list (rows of kv named by valid
// slots; zeros for invalid slots, so no stale or uninitialised LDS value can
// meet a zero probability).  It is read three ways:
//   * row-wise 16-byte reads (MFMA operands with the head dimension as the
//     contraction: K for S = Q K^T, V for dP = dO V^T);
//   * transposed 4-element reads (slot-major operands: V^T for O^T = V^T P^T,
//     K^T for dQ^T = K^T dS^T).
// Rows are padded by 16 bytes so that 16 consecutive rows start in distinct
// 4-bank groups (row-wise reads of one column chunk by 16 lanes are then free
// of bank conflicts).
#pragma once

#include "common.h"

namespace smla {

template <int DQK>
struct KvTile {
    static constexpr int RS = DQK + 8;           // row stride (elements)
    static constexpr int CH = DQK / 8;           // 16-byte chunks per row
    static constexpr int ELEMS = BLK * RS;

    // Slot -> KV row (or -1) for block b of token t, into s_row[0..BLK).
    __device__ static void load_rows(int* s_row, const int32_t* idx, int t, int W, int L,
                                     int S_kv, int b) {
        if (threadIdx.x < BLK) {
            s_row[threadIdx.x] = slot_row(idx, t, W, L, S_kv, b * BLK + (int)threadIdx.x);
        }
    }

    // Gather the rows named by s_row into the tile (256 threads).
    __device__ static void gather(__bf16* tile, const int* s_row, const __bf16* kv) {
        static_assert((BLK * CH) % 256 == 0, "gather assumes 256 threads");
#pragma unroll 6
        for (int it = 0; it < BLK * CH / 256; ++it) {
            const int id = it * 256 + (int)threadIdx.x;
            const int row = id / CH;
            const int ch = id - row * CH;
            const int r = s_row[row];
            u32x4 v = {0u, 0u, 0u, 0u};
            if (r >= 0) v = *reinterpret_cast<const u32x4*>(kv + (size_t)r * DQK + ch * 8);
            *reinterpret_cast<u32x4*>(tile + row * RS + ch * 8) = v;
        }
    }

    // Row-wise operand: rows m0 + (lane % 16), columns c0 + 8 * (lane / 16) .. +7.
    __device__ static bf16x8 row_op(const __bf16* tile, int m0, int c0, int lane) {
        return lds8(tile + (m0 + (lane & 15)) * RS + c0 + 8 * (lane >> 4));
    }

    // Transposed operand over slots: for lane group g = lane / 16 and column
    // c = c0 + lane % 16, the 8 values tile[s(g, j)][c], j = 0..7, where
    // s(g, j) = k0 + 4g + j for j < 4 and k0 + 16 + 4g + (j - 4) for j >= 4.
    // This is the slot order in which the C tile of an MFMA over two 16-slot
    // row tiles (slots k0..k0+15 and k0+16..k0+31) hands its values to lane
    // group g, so a C tile can be repacked into a B operand without moving
    // data across lanes.
    __device__ static bf16x8 slot_op(const __bf16* tile, int k0, int c0, int lane) {
        const int g = lane >> 4, w = lane & 15;
        const int row = k0 + 4 * g + (w >> 2);
        const int col = c0 + 4 * (w & 3);
        bf16x4 lo = lds_tr4(tile + row * RS + col);
        bf16x4 hi = lds_tr4(tile + (row + 16) * RS + col);
        return cat44(lo, hi);
    }
};

}  // namespace smla
