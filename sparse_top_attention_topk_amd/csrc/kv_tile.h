// The gathered KV tile in LDS: BLK top-k slots x d_qk bf16, one row per slot.
//
// Two layouts share one interface:
//   KvTile      rows padded by 16 bytes, filled through registers (zeros for
//               invalid slots);
//   KvTileSwz   unpadded rows with the 16-byte chunks of row r permuted by
//               chunk ^ f(r), filled by direct global->LDS loads (no
//               registers, asynchronous, so the next block's gather overlaps
//               the current block's math).  An invalid slot holds KV row 0
//               (finite data) and always meets a zero probability.
// Both are read two ways:
//   * row-wise 16-byte reads (MFMA operands whose contraction runs along d:
//     K for S = Q K^T, V for dP = dO V^T);
//   * transposed 4-element reads (slot-major operands: V^T for O^T = V^T P^T,
//     K^T for dQ^T = K^T dS^T).
// f(r) is chosen so that 16 consecutive rows read at one chunk column hit 16
// distinct 4-bank groups (row-wise reads), and 4 consecutive rows read as
// 32-byte pieces hit distinct 8-bank groups (transposed reads): with 64 banks
// of 4 bytes, a 1152-byte row starts 32 banks after the previous one and a
// 1024-byte row at the same bank.
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

template <int DQK>
struct SwzF;
template <>
struct SwzF<576> {
    __device__ static int f(int r) { return (((r >> 1) & 3) << 1) | ((r >> 3) & 1); }
};
template <>
struct SwzF<512> {
    __device__ static int f(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
};

template <int DQK>
struct KvTileSwz {
    static constexpr int CH = DQK / 8;           // 16-byte chunks per row
    static constexpr int ELEMS = BLK * DQK;
    static constexpr int ROWB = DQK * 2;         // row bytes
    static constexpr int INSTR = BLK * CH / 64;  // wave-wide 1 KB loads per tile
    // f(r) only involves r mod 16, and row tiles start at multiples of 16
    // rows, so every read of a lane sees one f.  The XOR then only permutes
    // the k-step index modulo NR (row-wise reads) or the column-tile index
    // modulo NS (transposed reads): NR / NS precomputed byte bases per lane
    // turn every operand read into base + immediate offset.
    static constexpr int NR = DQK == 576 ? 2 : 4;
    static constexpr int NS = DQK == 576 ? 4 : 8;

    __device__ static int f(int r) { return SwzF<DQK>::f(r); }

    // element offset of (row, col)
    __device__ static int at(int row, int col) {
        return row * DQK + ((((col >> 3) ^ f(row))) << 3) + (col & 7);
    }

    struct Lane {
        uint32_t rb[NR];   // row-wise reads: byte base for k-step ks % NR
        uint32_t sb[NS];   // transposed reads: byte base for column tile mc % NS
    };

    __device__ static Lane lane_bases(int lane) {
        Lane L;
        const int g = lane >> 4, w = lane & 15;
        {   // row-wise: row w, logical chunk 4 ks + g
            const int fr = f(w);
            const int b = fr >> 2, fl = fr & 3;
#pragma unroll
            for (int j = 0; j < NR; ++j)
                L.rb[j] = w * ROWB + 16 * (g ^ fl) + 64 * ((j ^ b) - j);
        }
        {   // transposed: row 4g + (w >> 2), column 16 mc + 4 (w & 3)
            const int row = 4 * g + (w >> 2);
            const int q = w & 3;
            const int fr = f(row);
            const int b2 = fr >> 1, f0 = fr & 1;
#pragma unroll
            for (int j = 0; j < NS; ++j)
                L.sb[j] = row * ROWB + 16 * ((q >> 1) ^ f0) + 8 * (q & 1) + 32 * ((j ^ b2) - j);
        }
        return L;
    }

    // Row-wise operand: rows m0 + lane % 16 (m0 a multiple of 16), logical
    // columns 32 ks + 8 (lane / 16) .. +7.
    __device__ static bf16x8 row_op(const __bf16* tile, const Lane& L, int m0, int ks) {
        const char* base = reinterpret_cast<const char*>(tile) + L.rb[ks % NR];
        return lds8(reinterpret_cast<const __bf16*>(base + m0 * ROWB + 64 * ks));
    }

    // Transposed operand over slots k0 .. k0+31 (k0 a multiple of 32), columns
    // 16 mc .. +15, in the slot order of KvTile::slot_op.
    __device__ static bf16x8 slot_op(const __bf16* tile, const Lane& L, int k0, int mc) {
        const char* base = reinterpret_cast<const char*>(tile) + L.sb[mc % NS] + k0 * ROWB + 32 * mc;
        bf16x4 lo = lds_tr4(reinterpret_cast<const __bf16*>(base));
        bf16x4 hi = lds_tr4(reinterpret_cast<const __bf16*>(base + 16 * ROWB));
        return cat44(lo, hi);
    }

    // Issue the direct global->LDS loads of the rows named by s_row (NW waves).
    // Wave w (a scalar) handles the 1 KB pieces w, w + NW, ...; lane l of
    // piece i fills chunk position 64 i + l of the tile.  Every position is
    // written: an invalid slot (s_row < 0) loads KV row 0, finite data that
    // the mask multiplies by a zero probability.  No wait here.
    template <int NW>
    __device__ static void gather_async(__bf16* tile, const int* s_row, const __bf16* kv,
                                        int wave_s, int lane) {
        static_assert(INSTR % NW == 0, "pieces must split evenly over the waves");
        // keep the per-piece index math inside the block loop (it is cheap)
        // instead of letting it be hoisted into many live registers
        int lv;
        asm volatile("v_mov_b32 %0, %1" : "=v"(lv) : "v"(lane));
        int rr[INSTR / NW];
        int off[INSTR / NW];
#pragma unroll
        for (int k = 0; k < INSTR / NW; ++k) {
            const int pos = (k * NW + wave_s) * 64 + lv;
            const int row = pos / CH;
            const int pc = pos - row * CH;
            rr[k] = s_row[row];
            off[k] = (pc ^ f(row)) << 3;
        }
#pragma unroll
        for (int k = 0; k < INSTR / NW; ++k) {
            const int r = rr[k] < 0 ? 0 : rr[k];
            const __bf16* src = kv + (size_t)r * DQK + off[k];
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             (lds_void*)(tile + (k * NW + wave_s) * 512), 16, 0, 0);
        }
    }
};

}  // namespace smla
