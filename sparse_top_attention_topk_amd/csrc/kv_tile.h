// The gathered KV tile in LDS: BLK top-k slots x d_qk bf16, one row per slot.
//
// Layout.  The first 512 columns of every row (all of V, most of K) form the
// main region, 64 rows of 1024 bytes at a stride of 1056 bytes; for
// d_qk = 576 the last 64 columns (the rotary part of K) form a rope region
// after it, 64 rows of 128 bytes in which 16-byte chunk c of row r is stored
// at position c ^ fr(r), fr(r) = 2 ((r >> 1) & 3).
//
// Why.  The gfx950 LDS has 64 banks of 4 bytes; measured with bank-conflict
// counters, a 16-byte-per-lane read (ds_read_b128) is served in four passes of
// 16 lanes {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}, and an
// 8-byte-per-lane read (ds_read_b64_tr_b16) in two passes of 32 lanes.  A pass
// costs one cycle when its lanes touch every bank once.  With the 32-byte row
// padding (and the rope permutation) every operand read below is
// conflict-free under that rule: row-wise 16-byte reads (MFMA operands that
// contract along d: K for S = Q K^T, V for dP = dO V^T) and transposed reads
// (slot-major operands: V^T for O^T = V^T P^T, K^T for dQ^T = K^T dS^T).  The
// main region needs no permutation, so its reads are a per-lane base plus an
// immediate offset.
//
// Filling.  The rows are gathered with 16-byte buffer loads that write LDS
// directly (no registers, asynchronous, so the next block's gather overlaps
// the current block's math).  A 1024-byte main row is one wave-wide load whose
// KV row offset is a scalar, so issuing a row costs a few scalar
// instructions.  The rope region is 8 loads of 8 rows x 128 bytes.  An
// invalid slot loads KV row 0 (finite data that always meets a zero
// probability).
#pragma once

#include "common.h"

namespace smla {

template <int DQK>
struct KvTileSwz {
    static_assert(DQK == 512 || DQK == 576, "d_qk must be 512 or 576");
    static constexpr bool ROPE = DQK == 576;
    static constexpr int MAIN_ROWB = 1056;                // main row stride (1024 bytes + 32 padding)
    static constexpr int ROPE_ROWB = 128;                 // bytes per rope row
    static constexpr int ROPE_OFF = BLK * MAIN_ROWB;      // byte offset of the rope region
    static constexpr int BYTES = ROPE_OFF + (ROPE ? BLK * ROPE_ROWB : 0);
    static constexpr int ELEMS = BYTES / 2;               // bf16 elements of LDS per tile
    static constexpr int KS_MAIN = 16;                    // k-steps of 32 columns in the main region
    static constexpr int MC_MAIN = 32;                    // 16-column tiles in the main region

    __device__ static int fr(int r) { return ((r >> 1) & 3) << 1; }

    // Per-lane byte bases.  Main-region reads are base + immediate.  The rope
    // permutation only depends on r mod 16 and every operand tile starts at a
    // multiple of 16 rows, so each lane sees one permutation per read, which
    // reduces to an XOR on the k-step (row-wise) or column-tile (transposed)
    // index.
    struct Lane {
        uint32_t mw;        // main row-wise base
        uint32_t sw;        // main transposed base
        uint32_t pw, px;    // rope row-wise: base, XOR on 64 * (ks - 16)
        uint32_t qw, qx;    // rope transposed: base, XOR on 32 * (mc - 32)
    };

    __device__ static Lane lane_bases(int lane) {
        Lane L;
        const int g = lane >> 4, w = lane & 15;
        // row-wise: row w, logical chunk 4 ks + g
        L.mw = w * MAIN_ROWB + 16 * g;
        const int h = fr(w);
        L.pw = ROPE_OFF + w * ROPE_ROWB + 16 * (g ^ (h & 3));
        L.px = (h >> 2) << 6;
        // transposed: row 4g + (w >> 2), column 16 mc + 4 (w & 3)
        const int row = 4 * g + (w >> 2);
        const int q = w & 3;
        L.sw = row * MAIN_ROWB + 16 * (q >> 1) + 8 * (q & 1);
        L.qw = ROPE_OFF + row * ROPE_ROWB + 16 * (q >> 1) + 8 * (q & 1);
        L.qx = (fr(row) >> 1) << 5;
        return L;
    }

    // Row-wise operand: rows m0 + lane % 16 (m0 a multiple of 16), logical
    // columns 32 ks + 8 (lane / 16) .. +7.  ks is a compile-time constant.
    __device__ static bf16x8 row_op(const __bf16* tile, const Lane& L, int m0, int ks) {
        const char* t = reinterpret_cast<const char*>(tile);
        if (!ROPE || ks < KS_MAIN)
            return lds8(reinterpret_cast<const __bf16*>(t + L.mw + m0 * MAIN_ROWB + 64 * ks));
        return lds8(reinterpret_cast<const __bf16*>(t + (((64u * (ks - KS_MAIN)) ^ L.px) + L.pw) +
                                                    m0 * ROPE_ROWB));
    }

    // Transposed operand over slots k0 .. k0+31 (k0 a multiple of 32), columns
    // 16 mc .. +15: for lane group g = lane / 16 and column c = 16 mc + lane % 16
    // the 8 values tile[s(g, j)][c], j = 0..7, with s(g, j) = k0 + 4g + j for
    // j < 4 and k0 + 16 + 4g + (j - 4) for j >= 4.  This is the slot order in
    // which the C tile of an MFMA over two 16-slot row tiles (slots k0..k0+15
    // and k0+16..k0+31) hands its values to lane group g, so a C tile can be
    // repacked into a B operand without moving data across lanes.
    // Main tiles mc < 32, rope tiles mc - 32 = 0..3; mc may be a run-time value.
    __device__ static bf16x8 slot_op(const __bf16* tile, const Lane& L, int k0, int mc) {
        if (ROPE && mc >= MC_MAIN) return slot_op_rope(tile, L, k0, mc - MC_MAIN);
        return slot_op_main(tile, L, k0, mc);
    }

    __device__ static bf16x8 slot_op_main(const __bf16* tile, const Lane& L, int k0, int mc) {
        const char* base = reinterpret_cast<const char*>(tile) + L.sw + k0 * MAIN_ROWB + 32 * mc;
        const bf16x4 lo = lds_tr4(reinterpret_cast<const __bf16*>(base));
        const bf16x4 hi = lds_tr4(reinterpret_cast<const __bf16*>(base + 16 * MAIN_ROWB));
        return cat44(lo, hi);
    }

    __device__ static bf16x8 slot_op_rope(const __bf16* tile, const Lane& L, int k0, int m) {
        const char* base = reinterpret_cast<const char*>(tile) + (((32u * m) ^ L.qx) + L.qw) + k0 * ROPE_ROWB;
        const bf16x4 lo = lds_tr4(reinterpret_cast<const __bf16*>(base));
        const bf16x4 hi = lds_tr4(reinterpret_cast<const __bf16*>(base + 16 * ROPE_ROWB));
        return cat44(lo, hi);
    }

    // ---- gather.  Buffer loads straight into LDS: the KV rows are addressed
    // through a buffer resource over kv, the KV row offset of a main row is a
    // scalar, the lane's chunk offset a vector register.  Row indices are
    // clamped into [0, S_kv) before use (load_row).
    __device__ static __amdgpu_buffer_rsrc_t kv_rsrc(const __bf16* kv, int S_kv) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kv), (short)0, S_kv * DQK * 2,
                                                 0x00020000);
    }

    // The same resource with live == false: zero records, so every load
    // through it is out of range (the range check covers the lane offset,
    // and any offset is >= 0 records) and reads no memory.  Used for the
    // gather after a row's last block, which would fill a free tile that
    // nobody reads: selecting the resource keeps the issuing loops free of
    // branches.
    __device__ static __amdgpu_buffer_rsrc_t kv_rsrc_if(const __bf16* kv, int S_kv, bool live) {
        return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(kv), (short)0,
                                                 live ? S_kv * DQK * 2 : 0, 0x00020000);
    }

    // NW waves split the 64 main rows: wave w owns rows w * RPW .. + RPW - 1.
    template <int NW>
    static constexpr int RPW = BLK / NW;

    // A slot row as a KV row to load: -1 (invalid slot) and anything outside
    // [0, S_kv) load row 0.  The main-row offset is a scalar offset, which the
    // buffer's range check does not cover, so every row stays in range here.
    __device__ static int load_row(int r, int S_kv) { return (unsigned)r < (unsigned)S_kv ? r : 0; }

    // Lane l of wave w holds the KV row of tile row w * RPW + l % RPW (invalid
    // slots -> row 0); lane i's value is read back as a scalar per row.
    template <int NW>
    __device__ static int row_ids(const int* s_row, int wave_s, int lane, int S_kv) {
        return load_row(s_row[wave_s * RPW<NW> + (lane & (RPW<NW> - 1))], S_kv);
    }

    // Issue main row i (a compile-time constant, 0 <= i < RPW) of this wave.
    template <int NW>
    __device__ static void gather_main_row(__bf16* tile, int ids, __amdgpu_buffer_rsrc_t rs, int wave_s,
                                           int lane, int i) {
        const int r = __builtin_amdgcn_readlane(ids, i);                  // scalar KV row
        const int row = wave_s * RPW<NW> + i;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (lds_void*)(reinterpret_cast<char*>(tile) + row * MAIN_ROWB), 16, lane << 4,
            r * (DQK * 2), 0, 0);
    }

    // Rope load k (0 <= k < 8 / NW) of this wave: rows 8j .. 8j+7 of the
    // rope region, j = k NW + wave, one 16-byte chunk per lane.
    template <int NW>
    __device__ static void gather_rope_one(__bf16* tile, const int* s_row, __amdgpu_buffer_rsrc_t rs,
                                           int wave_s, int lane, int k, int S_kv) {
        if constexpr (ROPE) {
            static_assert(NW <= 8 && 8 % NW == 0, "rope loads must split evenly");
            const int j = k * NW + wave_s;
            const int row = 8 * j + (lane >> 3);
            const int r = load_row(s_row[row], S_kv);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_void*)(reinterpret_cast<char*>(tile) + ROPE_OFF + 8 * j * ROPE_ROWB), 16,
                r * (DQK * 2) + 1024 + (((lane & 7) ^ fr(row)) << 4), 0, 0, 0);
        }
    }

    // All of this wave's rope loads (8 loads of 8 rows x 128 bytes, split
    // over the waves).
    template <int NW>
    __device__ static void gather_rope(__bf16* tile, const int* s_row, __amdgpu_buffer_rsrc_t rs,
                                       int wave_s, int lane, int S_kv) {
#pragma unroll
        for (int k = 0; k < 8 / NW; ++k) gather_rope_one<NW>(tile, s_row, rs, wave_s, lane, k, S_kv);
    }

    // The whole gather of one tile by this wave (the NW waves together fill
    // it).  No wait here.
    template <int NW>
    __device__ static void gather_async(__bf16* tile, const int* s_row, __amdgpu_buffer_rsrc_t rs,
                                        int wave_s, int lane, int S_kv) {
        const int ids = row_ids<NW>(s_row, wave_s, lane, S_kv);
#pragma unroll
        for (int i = 0; i < RPW<NW>; ++i) gather_main_row<NW>(tile, ids, rs, wave_s, lane, i);
        gather_rope<NW>(tile, s_row, rs, wave_s, lane, S_kv);
    }
};

}  // namespace smla
