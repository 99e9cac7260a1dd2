// Sparse MLA backward for gfx950.
//
// Method ([cuDNN-FE #785] Summary 1-3, Why 1-3, Not addressed; [cuDNN-FE
// #298]; [flash-attn #2882] Mechanism).  The probabilities are recomputed from
// the forward's LSE (no online softmax in the backward):
//   LSE_tot = glae(lse, sink)             (finite-max-guarded logaddexp)
//   P       = exp(S * scale - LSE_tot)    (invalid slots masked to 0 first)
//   dP      = dO V^T,  dS = P (dP - Delta)
//   dQ      = scale * dS K
//   dKV[idx] += scale * dS^T Q  (all d_qk columns) and P^T dO (first d_v)
//   d_sink  = -sum_t sigmoid(sink - lse) * Delta
//
// Kernels, in launch order (preprocess is its own entry point):
//   rows_count / rows_chunkscan / rows_scan / rows_parts / rows_fill
//                invert the index lists: every valid (token, slot) is listed
//                under its KV row, in token order (row r owns the segment
//                [off[r], off[r+1]) of the list, cut into parts of at most 64
//                entries); chunks of at most 16 tokens take rows_small, one
//                workgroup doing all of it
//   bwd_sdq      one workgroup per token and 64 heads: gathers each 64-slot
//                KV tile (async, double-buffered), recomputes S, P, dP, dS
//                with bf16 MFMA, stores P and scale*dS (bf16) to the workspace
//                and accumulates dQ^T = K^T (scale dS)^T in registers from the
//                same tile and the dS still in registers
//   dq_reduce    (block ranges split over several workgroups only) sums the
//                ranges' fp32 dQ shares in order
//   bwd_dkv      one workgroup per token: contracts over all heads,
//                u = (scale dS)^T q + P^T dO per valid slot (fp32 accumulate),
//                written to the slot's row of a [T * Wp] partial buffer in
//                16 bits per value (blocks of four values sharing the largest
//                exponent, 14-bit signed multiples of 2^-12 of it: error at
//                most 2^-13 of the block's largest magnitude, an order below
//                the bf16 rounding of P and dS that the MFMAs already see; the
//                partial traffic, which bounds this half of the backward, is
//                half that of fp32)
//   dkv_part / dkv_combine
//                sum each row's listed partials in token order, in bounded
//                parts (one wave each) and then per row; write dkv (rows no
//                valid slot names get 0)
//   dsink        one workgroup per head: sum over tokens in token order
// No fp32 atomics touch dkv: the scatter is a write of per-slot partials plus
// a streaming reduce.  A 64-slot block without a valid slot (the tail of a
// non-compact row) runs no math in bwd_sdq and bwd_dkv, and its P and dS are
// never stored or read: it would add exact zeros.  An empty row (no valid
// slot) is a uniform branch: dQ = 0 is written and the token's q, dO, lse and
// delta are not read.
#include "kv_tile.h"
#include "launch.h"

#include <type_traits>

namespace smla {

// ---------------------------------------------------------------------------
// Delta = rowsum(O * dO): one wave per (token, head) row of 512 values.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void preprocess_kernel(const __bf16* __restrict__ o,
                                                         const __bf16* __restrict__ dO,
                                                         float* __restrict__ delta, int rows) {
    const int row = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= rows) return;
    const size_t off = (size_t)row * 512 + lane * 8;
    const bf16x8 x = ld8_nt(o + off), y = ld8_nt(dO + off);
    float acc = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc += (float)x[j] * (float)y[j];
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 64);
    if (lane == 0) delta[row] = acc;
}

hipError_t launch_preprocess(const __bf16* o, const __bf16* dO, float* delta, int rows,
                             hipStream_t stream) {
    hipLaunchKernelGGL(preprocess_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, o, dO,
                       delta, rows);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Index inversion of one token chunk: its valid (token, slot) pairs grouped
// by KV row.  The chunk's tokens are cut into nsub sub-chunks of tchunk
// consecutive tokens.  rows_count counts, per sub-chunk, the valid slots
// naming each row (LDS counters, one workgroup per sub-chunk and range of
// INV_ROWS rows); rows_chunkscan and rows_scan turn the counts into row
// segments and per-sub-chunk offsets inside them; rows_fill walks each
// sub-chunk's tokens in order and appends every valid slot's local flat index
// (t - t0) * Wp + j to its row.  A row's list is therefore in token order,
// so the reduce sums each row in a fixed order: dKV does not depend on
// scheduling.  (Two slots of one token naming the same row carry identical
// contributions, so their relative order cannot change a sum.)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void fill_i32_kernel(int* __restrict__ p, int v, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256)
        p[i] = v;
}

// tokens [t_begin, t_end) of sub-chunk c and rows [r0, r0 + nr) of range blockIdx.y
struct InvPart {
    int t_begin, t_end, r0, nr;
    __device__ InvPart(const BwdArgs& a) {
        const int c = blockIdx.x;
        const int chunk_end = a.t0 + a.Tc;
        t_begin = a.t0 + c * a.tchunk;
        t_end = t_begin + a.tchunk < chunk_end ? t_begin + a.tchunk : chunk_end;
        r0 = (int)blockIdx.y * INV_ROWS;
        nr = a.S_kv - r0 < INV_ROWS ? a.S_kv - r0 : INV_ROWS;
    }
};

// The row of local slot i of a sub-chunk's token-major slot range (tokens
// t_begin ..), relative to r0, or -1 when the slot is not valid.  The index
// load is unconditional (i clamped into the range), so that several can be
// in flight.
// Branch-free row_length: the length load always happens (from the index
// array when there are no lengths), so a wait placed for one load does not
// cover the others in flight.
__device__ __forceinline__ int row_length_nb(const BwdArgs& a, int t) {
    const int32_t* p = a.len != nullptr ? a.len + t : a.idx;
    const int v = *p;
    const int L = v < 0 ? 0 : (v > a.W ? a.W : v);
    return a.len != nullptr ? L : a.W;
}

__device__ __forceinline__ int flat_slot_row(const BwdArgs& a, const InvPart& P, int i, int n) {
    const int ic = i < n ? i : n - 1;
    const int tl = ic / a.W;
    const int t = P.t_begin + tl, j = ic - tl * a.W;
    const int v = a.idx[(size_t)t * a.W + j];
    const int L = row_length_nb(a, t);
    return (i < n && j < L && v >= 0 && v < a.S_kv) ? v - P.r0 : -1;
}

__global__ __launch_bounds__(256) void rows_count_kernel(BwdArgs a) {
    extern __shared__ int s_cnt[];           // [nr]
    const InvPart P(a);
    for (int i = threadIdx.x; i < P.nr; i += 256) s_cnt[i] = 0;
    __syncthreads();
    // the sub-chunk's slots as one range, U index loads in flight per thread
    // (counting does not depend on the order)
    constexpr int U = 8;
    const int n = (P.t_end - P.t_begin) * a.W;
    for (int i0 = threadIdx.x; i0 < n; i0 += 256 * U) {
        int r[U];
#pragma unroll
        for (int u = 0; u < U; ++u) r[u] = flat_slot_row(a, P, i0 + 256 * u, n);
#pragma unroll
        for (int u = 0; u < U; ++u)
            if ((unsigned)r[u] < (unsigned)P.nr) atomicAdd(s_cnt + r[u], 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < P.nr; i += 256)
        a.chunk_cnt[(size_t)blockIdx.x * a.S_kv + P.r0 + i] = s_cnt[i];
}

// Per row: running offsets over the chunks (chunk_cnt becomes the exclusive
// prefix inside the row's segment) and the row total.  A workgroup takes 32
// rows; 8 threads per row scan 8 consecutive ranges of chunks and combine
// their sums through LDS (accesses of the 32 rows of a chunk are coalesced).
__global__ __launch_bounds__(256) void rows_chunkscan_kernel(BwdArgs a) {
    __shared__ int s_sum[8][32];
    const int rl = threadIdx.x & 31, part = threadIdx.x >> 5;
    const int r = (int)blockIdx.x * 32 + rl;
    const int nch = a.nsub;
    const int per = (nch + 7) / 8;
    const int c0 = part * per < nch ? part * per : nch;
    const int c1 = c0 + per < nch ? c0 + per : nch;
    // U counts in flight per thread in both passes
    constexpr int U = 8;
    int sum = 0;
    if (r < a.S_kv)
        for (int c = c0; c < c1; c += U) {
            int v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) v[u] = c + u < c1 ? a.chunk_cnt[(size_t)(c + u) * a.S_kv + r] : 0;
#pragma unroll
            for (int u = 0; u < U; ++u) sum += v[u];
        }
    s_sum[part][rl] = sum;
    __syncthreads();
    int run = 0;
    for (int q = 0; q < part; ++q) run += s_sum[q][rl];
    if (r >= a.S_kv) return;
    for (int c = c0; c < c1; c += U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = c + u < c1 ? a.chunk_cnt[(size_t)(c + u) * a.S_kv + r] : 0;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (c + u < c1) a.chunk_cnt[(size_t)(c + u) * a.S_kv + r] = run;
            run += v[u];
        }
    }
    if (part == 7) a.row_cnt[r] = run;
}

// Exclusive scans over the rows (one workgroup): row_off from the row totals,
// and part_off from the number of reduce parts of each row (a row's list is
// cut into parts of at most RPART entries, each summed by one wave).
constexpr int RPART = 64;

__device__ __forceinline__ int nparts(int cnt) { return (cnt + RPART - 1) / RPART; }

// Tiles of 8192 rows: thread i takes rows 8i .. 8i + 7 of the tile (two
// 16-byte loads, adjacent threads adjacent), the workgroup scans the
// per-thread sums (within each wave by shuffles, then over the 16 wave
// sums), and a carry runs from tile to tile.
__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
    }
    return v;
}

__global__ __launch_bounds__(1024) void rows_scan_kernel(BwdArgs a) {
    __shared__ int s_w[2][16];
    const int n = a.S_kv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    int carry = 0, carry2 = 0;
    for (int base = 0; base < n; base += 8192) {
        const int r0 = base + 8 * tid;
        int c[8];
        if (r0 + 8 <= n) {
            const u32x4 x = *reinterpret_cast<const u32x4*>(a.row_cnt + r0);
            const u32x4 y = *reinterpret_cast<const u32x4*>(a.row_cnt + r0 + 4);
#pragma unroll
            for (int k = 0; k < 4; ++k) { c[k] = (int)x[k]; c[4 + k] = (int)y[k]; }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) c[k] = r0 + k < n ? a.row_cnt[r0 + k] : 0;
        }
        int sum = 0, sum2 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) { sum += c[k]; sum2 += nparts(c[k]); }
        const int inc = wave_incl_scan(sum, lane), inc2 = wave_incl_scan(sum2, lane);
        if (lane == 63) { s_w[0][wave] = inc; s_w[1][wave] = inc2; }
        __syncthreads();
        int wpre = 0, wpre2 = 0, tot = 0, tot2 = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int v = s_w[0][w], v2 = s_w[1][w];
            if (w < wave) { wpre += v; wpre2 += v2; }
            tot += v; tot2 += v2;
        }
        int run = carry + wpre + inc - sum, run2 = carry2 + wpre2 + inc2 - sum2;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (r0 + k < n) {
                a.row_off[r0 + k] = run;
                a.part_off[r0 + k] = run2;
            }
            run += c[k];
            run2 += nparts(c[k]);
        }
        carry += tot;
        carry2 += tot2;
        __syncthreads();                       // s_w is reused by the next tile
    }
    if (tid == 0) {
        a.row_off[n] = carry;
        a.part_off[n] = carry2;
    }
}

// The whole inversion in one workgroup, for chunks of few slots (decode,
// short prefixes) where the five launches above are mostly launch latency:
// counts in LDS over all of the chunk's slots at once, the two exclusive
// scans with the part -> row map, then the row lists in token order (a
// barrier after each token; the next token's slot rows load while the
// current one is placed).  Same lists, offsets and parts as the five kernels.
// Needs S_kv <= INV_ROWS (the counters in LDS) and W <= SMALL_INV_W; taken
// for at most SMALL_INV_TOKENS tokens (each token costs a barrier: measured,
// 64 tokens of 32 slots took 31 us here against 20 us in the five kernels,
// one token of 1152 slots 24 against 53 us, 16 tokens 46 against 57 us).
constexpr int SMALL_INV_TOKENS = 16;
constexpr int SMALL_INV_W = 4096;            // slots of a token held by the 1024 threads

__global__ __launch_bounds__(1024) void rows_small_kernel(BwdArgs a) {
    extern __shared__ int s_c[];             // [S_kv]: counts, then cursors
    __shared__ int s_w[2][16];
    const int n = a.S_kv;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < n; i += 1024) s_c[i] = 0;
    __syncthreads();
    {
        const int total = a.Tc * a.W;
        for (int i0 = 0; i0 < total; i0 += 4 * 1024) {
            int r[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * 1024 + tid;
                const int tl = i / a.W;
                const int t = a.t0 + (tl < a.Tc ? tl : a.Tc - 1);
                r[u] = i < total ? slot_row(a.idx, t, a.W, row_length(a.len, t, a.W), n, i - tl * a.W) : -1;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (r[u] >= 0) atomicAdd(s_c + r[u], 1);
        }
    }
    __syncthreads();
    // tiles of 8192 rows, 8 per thread (as rows_scan_kernel, from LDS)
    int carry = 0, carry2 = 0;
    for (int base = 0; base < n; base += 8192) {
        const int r0 = base + 8 * tid;
        int c[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) c[k] = r0 + k < n ? s_c[r0 + k] : 0;
        int sum = 0, sum2 = 0;
#pragma unroll
        for (int k = 0; k < 8; ++k) { sum += c[k]; sum2 += nparts(c[k]); }
        const int inc = wave_incl_scan(sum, lane), inc2 = wave_incl_scan(sum2, lane);
        if (lane == 63) { s_w[0][wave] = inc; s_w[1][wave] = inc2; }
        __syncthreads();
        int wpre = 0, wpre2 = 0, tot = 0, tot2 = 0;
#pragma unroll
        for (int w = 0; w < 16; ++w) {
            const int v = s_w[0][w], v2 = s_w[1][w];
            if (w < wave) { wpre += v; wpre2 += v2; }
            tot += v; tot2 += v2;
        }
        int run = carry + wpre + inc - sum, run2 = carry2 + wpre2 + inc2 - sum2;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (r0 + k < n) {
                a.row_off[r0 + k] = run;
                a.part_off[r0 + k] = run2;
                s_c[r0 + k] = run;                   // the row's cursor
                for (int q = 0; q < nparts(c[k]); ++q) a.part_row[run2 + q] = r0 + k;
            }
            run += c[k];
            run2 += nparts(c[k]);
        }
        carry += tot;
        carry2 += tot2;
        __syncthreads();                       // s_w is reused by the next tile
    }
    if (tid == 0) {
        a.row_off[n] = carry;
        a.part_off[n] = carry2;
    }
    // slots j = tid + 1024 u of token t (u < 4 covers W <= SMALL_INV_W)
    auto rows_of = [&](int t, int (&r)[4]) {
        const int L = row_length(a.len, t, a.W);
#pragma unroll
        for (int u = 0; u < 4; ++u) r[u] = slot_row(a.idx, t, a.W, L, n, u * 1024 + tid);
    };
    int cur[4], nxt[4] = {-1, -1, -1, -1};
    rows_of(a.t0, cur);
    for (int t = a.t0; t < a.t0 + a.Tc; ++t) {
        if (t + 1 < a.t0 + a.Tc) rows_of(t + 1, nxt);
#pragma unroll
        for (int u = 0; u < 4; ++u)
            if (cur[u] >= 0) a.entries[atomicAdd(s_c + cur[u], 1)] = (t - a.t0) * a.Wp + u * 1024 + tid;
        __syncthreads();                       // token order
#pragma unroll
        for (int u = 0; u < 4; ++u) cur[u] = nxt[u];
    }
}

// part -> row map for the reduce
__global__ __launch_bounds__(256) void rows_parts_kernel(BwdArgs a) {
    const int r = (int)blockIdx.x * 256 + threadIdx.x;
    if (r >= a.S_kv) return;
    for (int p = a.part_off[r]; p < a.part_off[r + 1]; ++p) a.part_row[p] = r;
}

// rows_fill's token loop for W <= 256 NJ: a token's slots in registers
// (slot k * 256 + tid), raw indices and length in two register sets taken in
// turn, so that the next token's loads stay in flight while the current one
// is placed (validity is decided at use); the barrier between tokens waits
// for the LDS cursors only.  The loads are not under a branch (past the
// sub-chunk's last token they reload it, unused), and the length goes
// through a lane-dependent address: moved to a scalar register at once, it
// would be waited for right where it is issued.
template <int NJ>
__device__ __forceinline__ void fill_tokens(const BwdArgs& a, const InvPart& P, int* s_cur) {
    int lane_zero;
    asm volatile("v_mov_b32 %0, 0" : "=v"(lane_zero));
    auto load_token = [&](int t, int (&v)[NJ], int& len_raw) {
        len_raw = *(a.len != nullptr ? a.len + t + lane_zero : a.idx + lane_zero);
#pragma unroll
        for (int k = 0; k < NJ; ++k) {
            const int j = k * 256 + (int)threadIdx.x;
            v[k] = a.idx[(size_t)t * a.W + (j < a.W ? j : a.W - 1)];
        }
    };
    auto place = [&](int t, const int (&v)[NJ], int len_raw) {
        const int L = a.len != nullptr ? (len_raw < 0 ? 0 : (len_raw > a.W ? a.W : len_raw)) : a.W;
#pragma unroll
        for (int k = 0; k < NJ; ++k) {
            const int j = k * 256 + (int)threadIdx.x;
            const int r = (j < L && v[k] >= 0 && v[k] < a.S_kv) ? v[k] - P.r0 : -1;
            if ((unsigned)r < (unsigned)P.nr) a.entries[atomicAdd(s_cur + r, 1)] = (t - a.t0) * a.Wp + j;
        }
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");   // token order within the sub-chunk
    };
    const int t_last = P.t_end - 1;
    int va[NJ], vb[NJ], la, lb;
    load_token(P.t_begin, va, la);
    for (int t = P.t_begin; t < P.t_end; t += 2) {
        load_token(t + 1 < t_last ? t + 1 : t_last, vb, lb);
        place(t, va, la);
        if (t + 1 >= P.t_end) break;
        load_token(t + 2 < t_last ? t + 2 : t_last, va, la);
        place(t + 1, vb, lb);
    }
}

__global__ __launch_bounds__(256) void rows_fill_kernel(BwdArgs a) {
    extern __shared__ int s_cur[];           // [nr]
    const InvPart P(a);
    {
        const int* ro = a.row_off + P.r0;
        const int* cc = a.chunk_cnt + (size_t)blockIdx.x * a.S_kv + P.r0;
        for (int i0 = 0; i0 < P.nr; i0 += 8 * 256) {
            int v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                // unconditional loads (index clamped): all 16 in flight
                const int i = i0 + k * 256 + (int)threadIdx.x;
                const int ic = i < P.nr ? i : P.nr - 1;
                v[k] = ro[ic] + cc[ic];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int i = i0 + k * 256 + (int)threadIdx.x;
                if (i < P.nr) s_cur[i] = v[k];
            }
        }
    }
    __syncthreads();
    if (a.W <= 4 * 256) {
        fill_tokens<4>(a, P, s_cur);
        return;
    }
    if (a.W <= 8 * 256) {
        fill_tokens<8>(a, P, s_cur);
        return;
    }
    for (int t = P.t_begin; t < P.t_end; ++t) {
        const int L = row_length(a.len, t, a.W);
        for (int j = threadIdx.x; j < L; j += 256) {
            const int r = slot_row(a.idx, t, a.W, L, a.S_kv, j) - P.r0;
            if ((unsigned)r < (unsigned)P.nr) a.entries[atomicAdd(s_cur + r, 1)] = (t - a.t0) * a.Wp + j;
        }
        __syncthreads();                     // token order within the sub-chunk
    }
}

__device__ __forceinline__ int raw_index_b(const BwdArgs& a, int t, int j) {
    return a.idx[(size_t)t * a.W + (j < a.W ? j : a.W - 1)];
}

__device__ __forceinline__ int valid_row_b(int v, int j, int L, int S_kv) {
    return (j < L && v >= 0 && v < S_kv) ? v : -1;
}

// The double-buffered gather loop of the kernels that gather KV tiles:
// body(tile, rows, b, gs, live) runs block b from tile 0 (even b) or tile 1
// (odd b) and issues, spread over its math (GatherSpread), this wave's share
// of the gather of block b + 1 from the slot rows grows into the other tile
// gtile (the last block issues none).

// The next block's gather, one load per step of a matrix loop: main rows at
// steps 0 .. RPW - 1, rope loads at the steps after (a 1 KB row load takes
// the address unit about 20 cycles; issued back to back they stall the wave,
// between MFMAs they cost almost nothing).
template <int DQK, int NW>
struct GatherSpread {
    using Tile = KvTileSwz<DQK>;
    static constexpr int RPW = Tile::template RPW<NW>;
    static constexpr int STEPS = RPW + (Tile::ROPE ? 8 / NW : 0);
    __bf16* gtile;
    const int* grows;
    __amdgpu_buffer_rsrc_t kvr;      // zero records when there is no next block: no memory read
    int ids, wave, lane, s_kv;
    __device__ GatherSpread(__bf16* gt, const int* gr, const __bf16* kv, int w, int l, int S_kv, bool next)
        : gtile(gt), grows(gr), kvr(Tile::kv_rsrc_if(kv, S_kv, next)),
          ids(Tile::template row_ids<NW>(gr, w, l, S_kv)), wave(w), lane(l), s_kv(S_kv) {}
    // step is a compile-time constant after unrolling
    __device__ void step(int s) const {
        if (s < RPW) Tile::template gather_main_row<NW>(gtile, ids, kvr, wave, lane, s);
        else if (s < STEPS) Tile::template gather_rope_one<NW>(gtile, grows, kvr, wave, lane, s - RPW, s_kv);
    }
    __device__ void all() const { Tile::template gather_async<NW>(gtile, grows, kvr, wave, lane, s_kv); }
};

// post() runs once, right after the first block's gather is issued: work that
// waits for its own loads there overlaps them with that gather.  early() runs
// once, right after the loads of the row's first indices are issued and
// before they are waited for: loads it issues travel with them (they complete
// in issue order, so the wait for the indices does not wait for them).
struct NoPost {
    __device__ void operator()() const {}
};

// The blocks a workgroup of the split kernels runs: [b_lo, ...) with slots
// below j_hi (the whole row without a split).
struct BlockRange {
    int b_lo, j_hi;
};

__device__ __forceinline__ BlockRange block_range(const BwdArgs& a, int L) {
    if (a.nsplit <= 1) return {0, L};
    const int b_lo = (int)blockIdx.z * a.bps;
    const int j_end = (b_lo + a.bps) * BLK;
    return {b_lo, L < j_end ? L : j_end};
}

template <int DQK, int NW, typename Body, typename Post = NoPost, typename Early = NoPost>
__device__ __forceinline__ void gathered_blocks(const BwdArgs& a, __bf16* s_tile0, __bf16* s_tile1,
                                                int (*s_rows)[BLK], int* s_live, int* s_last, int t, int nblk,
                                                BlockRange rg, int wave, int lane, Body&& body, Post&& post = Post{},
                                                Early&& early = Early{}) {
    const int b_lo = rg.b_lo, j_hi = rg.j_hi;
    using Tile = KvTileSwz<DQK>;
    const auto kvr = Tile::kv_rsrc(a.kv, a.S_kv);
    const int tid = threadIdx.x;
    // The row's last valid slot: the blocks after its block hold padding only
    // (the tail of a non-compact row) and are not run.  The raw indices of the
    // range's first 4 x NW x 64 slots (which hold the first two blocks: the
    // slot rows of block b_lo are v[0] of threads 0..63) and of block
    // b_lo + 1 go out in one batch, then early()'s loads behind them.
    {
        constexpr int NTH = NW * 64;
        static_assert(NTH >= 2 * BLK, "the first index batch must cover two blocks");
        const int j_first = b_lo * BLK;
        int v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = raw_index_b(a, t, j_first + k * NTH + tid);
        const int r1 = raw_index_b(a, t, j_first + BLK + (tid & (BLK - 1)));
        __builtin_amdgcn_sched_barrier(0);
        early();
        __builtin_amdgcn_sched_barrier(0);
        int last = -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = j_first + k * NTH + tid;
            if (valid_row_b(v[k], j, j_hi, a.S_kv) >= 0) last = j;
        }
        for (int j0 = j_first + 4 * NTH; j0 < j_hi; j0 += 4 * NTH) {     // rows longer than one batch
            int u[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) u[k] = raw_index_b(a, t, j0 + k * NTH + tid);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = j0 + k * NTH + tid;
                if (valid_row_b(u[k], j, j_hi, a.S_kv) >= 0) last = j;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) last = max(last, __shfl_xor(last, m, 64));
        if (lane == 0) s_last[wave] = last;
        if (tid < BLK) {
            put_rows(s_rows[0], &s_live[0], valid_row_b(v[0], j_first + tid, j_hi, a.S_kv), tid);
            put_rows(s_rows[1], &s_live[1], valid_row_b(r1, j_first + BLK + tid, j_hi, a.S_kv), tid);
            put_rows(s_rows[2], &s_live[2], -1, tid);    // written again before any block reads it
        }
    }
    __syncthreads();
    int last = s_last[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) last = max(last, s_last[w]);
    const int nbr = nblk;                                   // blocks of the row
    nblk = __builtin_amdgcn_readfirstlane(last < 0 ? 0 : last / BLK + 1 - b_lo);   // blocks of the range
    if (nbr > 0) {
        if (nblk > 0) Tile::template gather_async<NW>(s_tile0, s_rows[0], kvr, wave, lane, a.S_kv);
        post();
    }
    // Block k: wait for its tile; store the slot rows of block k + 1 (their
    // raw indices were loaded at block k - 1, and the wait just covered that
    // load: storing them any earlier would wait for the whole gather issued
    // since); load the raw indices of block k + 2; run the body, which issues
    // the gather of block k + 1.
    int ahead = 0;
    for (int b = 0; b < nblk; b += 2) {
        wait_vmem();
        if (b > 0 && b + 1 < nblk && tid < BLK)
            put_rows(s_rows[(b + 1) % 3], &s_live[(b + 1) % 3],
                     valid_row_b(ahead, (b_lo + b + 1) * BLK + tid, j_hi, a.S_kv), tid);
        __syncthreads();
        ahead = tid < BLK ? raw_index_b(a, t, (b_lo + b + 2) * BLK + tid) : 0;
        __builtin_amdgcn_sched_barrier(0);
        body(s_tile0, s_rows[b % 3], b_lo + b,
             GatherSpread<DQK, NW>(s_tile1, s_rows[(b + 1) % 3], a.kv, wave, lane, a.S_kv, b + 1 < nblk),
             __builtin_amdgcn_readfirstlane(s_live[b % 3]) != 0);
        if (b + 1 >= nblk) break;
        wait_vmem();
        if (b + 2 < nblk && tid < BLK)
            put_rows(s_rows[(b + 2) % 3], &s_live[(b + 2) % 3],
                     valid_row_b(ahead, (b_lo + b + 2) * BLK + tid, j_hi, a.S_kv), tid);
        __syncthreads();
        ahead = tid < BLK ? raw_index_b(a, t, (b_lo + b + 3) * BLK + tid) : 0;
        __builtin_amdgcn_sched_barrier(0);
        body(s_tile1, s_rows[(b + 1) % 3], b_lo + b + 1,
             GatherSpread<DQK, NW>(s_tile0, s_rows[(b + 2) % 3], a.kv, wave, lane, a.S_kv, b + 2 < nblk),
             __builtin_amdgcn_readfirstlane(s_live[(b + 1) % 3]) != 0);
    }
    wait_vmem();
}

// ---------------------------------------------------------------------------
// delta_exact: Delta = sum_j P_j dP_j per head over the token's valid slots,
// fp32, from the same S^T = K Q^T and dP^T = V dO^T as the backward (NW waves
// x NT x 16 heads).  q and dO stay in registers as the B operands.  Per
// 64-slot block, two halves of 32 slots.
// ---------------------------------------------------------------------------
template <int DQK, int NW, int NT>
__device__ __forceinline__ void delta_exact_block(const BwdArgs& a, const __bf16* tile,
                                                  const typename KvTileSwz<DQK>::Lane& TL, const int* rows,
                                                  const bf16x8 (&qop)[NT][DQK / 32],
                                                  const bf16x8 (&dop)[NT][16], const float (&lse2)[NT],
                                                  float (&pdp)[NT], int lane, const GatherSpread<DQK, NW>& gs) {
    using Tile = KvTileSwz<DQK>;
    constexpr int KS = DQK / 32, KV_ = 16;
    static_assert(GatherSpread<DQK, NW>::STEPS <= KS, "the gather must fit in the first half's S loop");
    const int g = lane >> 4;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
        f32x4 sacc[2][NT], dpacc[2][NT];
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) { sacc[m][nt] = zero4(); dpacc[m][nt] = zero4(); }
        bf16x8 kop[2][2];
#pragma unroll
        for (int m = 0; m < 2; ++m) kop[0][m] = Tile::row_op(tile, TL, (2 * half + m) * 16, 0);
        // k-steps 0..KS-1 feed S; the first 16 (the V columns) also feed dP
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < KS) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    kop[cur ^ 1][m] = Tile::row_op(tile, TL, (2 * half + m) * 16, ks + 1);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    sacc[m][nt] = mfma16(kop[cur][m], qop[nt][ks], sacc[m][nt]);
                    if (ks < KV_) dpacc[m][nt] = mfma16(kop[cur][m], dop[nt][ks], dpacc[m][nt]);
                }
            if (half == 0) gs.step(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
        // P = 2^(s * scale * log2 e - LSE_tot * log2 e), masked; sum P dP
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const bool ok = rows[(2 * half + m) * 16 + 4 * g + i] >= 0;
                    const float p = ok ? fast_exp2(sacc[m][nt][i] * a.scale_log2 - lse2[nt]) : 0.f;
                    pdp[nt] = __builtin_fmaf(p, dpacc[m][nt][i], pdp[nt]);
                }
    }
}

// Delta = sum over the d_v columns of O dO in fp32 (the preprocess pass's
// arithmetic, fused into the backward's S/dP pass): lane (g, n) takes columns
// 32 ks + 8g .. +7 of head h_wave + 16 nt + n (the layout of the dO operands,
// which dO_at(nt, ks, row) returns), then the four lane groups are summed.
// Writes delta_out for the existing heads and returns the sums in dlt.
template <int NT, typename DOAt>
__device__ __forceinline__ void fused_delta(const BwdArgs& a, int t, int h_wave, int lane, DOAt&& dO_at,
                                            float (&dlt)[NT]) {
    const int g = lane >> 4, n = lane & 15;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int head = h_wave + nt * 16 + n;
        const bool hv = head < a.H;
        const size_t row = (size_t)t * a.H + (hv ? head : 0);
        float acc = 0.f;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const bf16x8 x = hv ? ld8(a.o + row * 512 + 32 * ks + 8 * g) : zero8();
            const bf16x8 y = hv ? dO_at(nt, ks, row) : zero8();
#pragma unroll
            for (int j = 0; j < 8; ++j) acc += (float)x[j] * (float)y[j];
        }
        acc += __shfl_xor(acc, 16, 64);
        acc += __shfl_xor(acc, 32, 64);
        dlt[nt] = acc;
        if (hv && g == 0) a.delta_out[row] = acc;
    }
}

template <int DQK, int NW, int NT>
__global__ __launch_bounds__(NW * 64, 1) void delta_exact_kernel(BwdArgs a) {
    using Tile = KvTileSwz<DQK>;
    constexpr int KS = DQK / 32, HT = NW * NT * 16;
    __shared__ __attribute__((aligned(16))) __bf16 s_tile0[Tile::ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 s_tile1[Tile::ELEMS];
    __shared__ int s_rows[3][BLK];
    __shared__ int s_live[3];
    __shared__ int s_last[NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    const int t = a.t0 + a.Tc - 1 - (int)blockIdx.x;     // the longest rows first
    const int h_wave = (int)blockIdx.y * HT + wave * NT * 16;
    const bool active = h_wave < a.H;
    const int L = row_length(a.len, t, a.W);
    const int nblk = (L + BLK - 1) / BLK;
    if (nblk == 0) {                             // uniform: Delta of an empty row is 0
        if (g == 0)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const int head = h_wave + nt * 16 + n;
                if (head < a.H) a.delta_out[(size_t)t * a.H + head] = 0.f;
            }
        return;
    }

    // The LSE and sink scalars load first; q and dO go out right behind the
    // row's first indices (early), unconditionally (lanes of heads past H
    // read head 0's row and zero it: the compiler loses count of loads issued
    // inside a branch), so that the wait for those indices does not wait for
    // them; the LSE arithmetic waits until the first tile's gather is in
    // flight (post).
    bf16x8 qop[NT][KS], dop[NT][16];
    float lse2[NT], l_raw[NT], sk_raw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int head = h_wave + nt * 16 + n;
        const bool hv = head < a.H;
        l_raw[nt] = a.lse[(size_t)t * a.H + (hv ? head : 0)];
        sk_raw[nt] = a.sink ? a.sink[hv ? head : 0] : 0.f;
    }
    auto early = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int head = h_wave + nt * 16 + n;
            const bool hv = head < a.H;
            const size_t row = (size_t)t * a.H + (hv ? head : 0);
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const bf16x8 x = ld8(a.dO + row * 512 + 32 * ks + 8 * g);
                dop[nt][ks] = hv ? x : zero8();
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 x = ld8(a.q + row * DQK + 32 * ks + 8 * g);
                qop[nt][ks] = hv ? x : zero8();
            }
        }
    };
    auto post = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const bool hv = h_wave + nt * 16 + n < a.H;
            // +inf for a saturating sink: every P is 0
            lse2[nt] = hv ? (a.sink ? glae(l_raw[nt], sk_raw[nt]) : l_raw[nt]) * LOG2E : 0.f;
        }
    };
    float pdp[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) pdp[nt] = 0.f;
    const typename Tile::Lane TL = Tile::lane_bases(lane);
    gathered_blocks<DQK, NW>(a, s_tile0, s_tile1, s_rows, s_live, s_last, t, nblk, block_range(a, L),
                             wave, lane,
                             [&](const __bf16* tile, const int* rows, int, const auto& gs, bool live) {
                                 if (active && live)
                                     delta_exact_block<DQK, NW, NT>(a, tile, TL, rows, qop, dop, lse2, pdp, lane,
                                                                    gs);
                                 else
                                     gs.all();
                             }, post, early);
    // lanes (g, n), g = 0..3, hold slot subsets of head n: sum them
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        float v = pdp[nt];
        v += __shfl_xor(v, 16, 64);
        v += __shfl_xor(v, 32, 64);
        const int head = h_wave + nt * 16 + n;
        if (active && g == 0 && head < a.H) a.delta_out[(size_t)t * a.H + head] = v;
    }
}

// dQ of a split backward: the splits' fp32 shares summed in split order, one
// wave per (token, head), rounded to bf16.
template <int DQK>
__global__ __launch_bounds__(256) void dq_reduce_kernel(BwdArgs a) {
    const int row = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.Tc * a.H) return;
    const int tl = row / a.H, h = row - tl * a.H;
    const float* src = a.dq_part + ((size_t)tl * a.nsplit * a.H + h) * DQK;    // split s: + s * H * DQK
    const size_t sstride = (size_t)a.H * DQK;
    for (int c = 4 * lane; c < DQK; c += 256) {
        f32x4 acc = zero4();
        int s = 0;
        for (; s + 4 <= a.nsplit; s += 4) {          // four shares in flight, summed in split order
            f32x4 x[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = *reinterpret_cast<const f32x4*>(src + (s + k) * sstride + c);
#pragma unroll
            for (int k = 0; k < 4; ++k) acc += x[k];
        }
        for (; s < a.nsplit; ++s) acc += *reinterpret_cast<const f32x4*>(src + s * sstride + c);
        st4(a.dq + ((size_t)(a.t0 + tl) * a.H + h) * DQK + c, cvt4(acc[0], acc[1], acc[2], acc[3]));
    }
}

// Two 8-byte pieces x0, x1 in each of the lanes (g, n), g = 0..3, of one row n:
// piece m of lane g covers elements 16 m + 4 g .. +3 of a 32-element stretch.
// Afterwards lane g holds elements 8 g .. 8 g + 7 (x0 the first four), so the
// stretch goes out as one 16-byte store per lane.  Two swap steps between
// 16-lane rows: rows 2, 3 of x0 with rows 0, 1 of x1, then rows 1, 3 of x0
// with rows 0, 2 of x1.
__device__ __forceinline__ void transpose_pairs(u32x2& x0, u32x2& x1) {
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const auto x = __builtin_amdgcn_permlane32_swap(x0[w], x1[w], false, false);
        x0[w] = x[0];
        x1[w] = x[1];
    }
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const auto x = __builtin_amdgcn_permlane16_swap(x0[w], x1[w], false, false);
        x0[w] = x[0];
        x1[w] = x[1];
    }
}

// ---------------------------------------------------------------------------
// bwd_sdq: S, P, dP, dS and dQ of 64 heads of one token in one pass over the
// token's gathered blocks.  Four waves of 16 heads, one per SIMD: q and dO
// (the B operands of S^T = K Q^T and dP^T = V dO^T) and the dQ^T accumulators
// of all d_qk columns take about 300 registers per lane.  Per half block (32
// slots) the wave forms P and scale dS in the C layout of its two 16-slot
// S^T tiles, stores them for the dKV pass, and uses the same registers,
// rounded to bf16, as the B operand of dQ^T += K^T (scale dS)^T: that C
// layout is the slot order of KvTileSwz::slot_op, so dS reaches the dQ
// product without a trip through LDS or memory, and the gathered tile serves
// both products.  More than 64 heads take more workgroups per token
// (blockIdx.y).
// ---------------------------------------------------------------------------
template <int DQK>
__device__ __forceinline__ void sdq_block(const BwdArgs& a, const __bf16* tile,
                                          const typename KvTileSwz<DQK>::Lane& TL, const int* rows,
                                          const bf16x8 (&qop)[DQK / 32], const bf16x8 (&dop)[16], float lse2,
                                          float dlt, f32x4 (&acc)[DQK / 16], int t, int head, int b, int lane,
                                          const GatherSpread<DQK, 4>& gs) {
    using Tile = KvTileSwz<DQK>;
    constexpr int KS = DQK / 32, KV_ = 16, MC = DQK / 16;
    static_assert(GatherSpread<DQK, 4>::STEPS <= KS, "the gather must fit in the first half's S loop");
    const int g = lane >> 4;
    const bool hv = head < a.H;

    // The halves in the order S(0), S(1), dQ(0), dQ(1): the P / dS arithmetic
    // of half 0 runs between the MFMAs of S(1) and that of half 1 between
    // those of dQ(0), so that it overlaps matrix work (one wave per SIMD:
    // nothing else would).  Each half's arithmetic and its order are unchanged.
    f32x4 sacc[2][2], dpacc[2][2];              // [half][m]
    // ok[h][k]: slot 32 h + 16 (k / 4) + 4g + k % 4 is valid (each half's
    // flags are read from LDS right before that half's P / dS steps)
    bool ok[2][8];
    auto flags = [&](auto H) {
        constexpr int h = decltype(H)::value;
#pragma unroll
        for (int k = 0; k < 8; ++k) ok[h][k] = rows[(2 * h + (k >> 2)) * 16 + 4 * g + (k & 3)] >= 0;
    };

    // S^T and dP^T for slots 32 h .. +31 (K operands two k-steps ahead: one
    // wave per SIMD leaves the LDS latency to the wave's own prefetch); the
    // first 16 k-steps (the V columns) also feed dP; step(ks) runs after each
    // k-step's MFMAs
    auto s_loop = [&](auto H, auto&& step) {
        constexpr int h = decltype(H)::value;
#pragma unroll
        for (int m = 0; m < 2; ++m) { sacc[h][m] = zero4(); dpacc[h][m] = zero4(); }
        constexpr int SA = 2;
        bf16x8 kop[SA + 1][2];
#pragma unroll
        for (int k = 0; k < SA; ++k)
#pragma unroll
            for (int m = 0; m < 2; ++m) kop[k][m] = Tile::row_op(tile, TL, (2 * h + m) * 16, k);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            if (ks + SA < KS) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    kop[(ks + SA) % (SA + 1)][m] = Tile::row_op(tile, TL, (2 * h + m) * 16, ks + SA);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m) {
                sacc[h][m] = mfma16(kop[ks % (SA + 1)][m], qop[ks], sacc[h][m]);
                if (ks < KV_) dpacc[h][m] = mfma16(kop[ks % (SA + 1)][m], dop[ks], dpacc[h][m]);
            }
            step(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // value k (0..7) of half h: P = 2^(s * scale * log2 e - LSE_tot * log2 e),
    // masked; dS' = scale P (dP - Delta).  P replaces S, dS' replaces dP.
    auto epi_step = [&](auto H, int k) {
        constexpr int h = decltype(H)::value;
        const int m = k >> 2, i = k & 3;
        const float p = ok[h][k] ? fast_exp2(sacc[h][m][i] * a.scale_log2 - lse2) : 0.f;
        sacc[h][m][i] = p;
        dpacc[h][m][i] = p * (dpacc[h][m][i] - dlt) * a.scale;
    };

    // bf16 P and dS' of half h: stored for the dKV pass; dS' returned as the B
    // operand of dQ^T (lane (g, n) holds slots 32 h + 4g + j and
    // 32 h + 16 + 4g + j of head n, the order of slot_op).  For the stores the
    // pieces are regrouped over g (transpose_pairs): lane (g, n) writes slots
    // 32 h + 8g .. +7 of head n, 16 bytes, into P and into dS'.
    auto finish = [&](auto H) {
        constexpr int h = decltype(H)::value;
        const bf16x4 ds_lo = cvt4(dpacc[h][0][0], dpacc[h][0][1], dpacc[h][0][2], dpacc[h][0][3]);
        const bf16x4 ds_hi = cvt4(dpacc[h][1][0], dpacc[h][1][1], dpacc[h][1][2], dpacc[h][1][3]);
        u32x2 p0 = __builtin_bit_cast(u32x2, cvt4(sacc[h][0][0], sacc[h][0][1], sacc[h][0][2], sacc[h][0][3]));
        u32x2 p1 = __builtin_bit_cast(u32x2, cvt4(sacc[h][1][0], sacc[h][1][1], sacc[h][1][2], sacc[h][1][3]));
        u32x2 d0 = __builtin_bit_cast(u32x2, ds_lo), d1 = __builtin_bit_cast(u32x2, ds_hi);
        transpose_pairs(p0, p1);
        transpose_pairs(d0, d1);
        if (hv) {
            const size_t base = ((size_t)(t - a.t0) * a.H + head) * a.Wp + b * BLK + h * 32 + 8 * g;
            *reinterpret_cast<u32x4*>(a.ws_p + base) = u32x4{p0[0], p0[1], p1[0], p1[1]};
            *reinterpret_cast<u32x4*>(a.ws_ds + base) = u32x4{d0[0], d0[1], d1[0], d1[1]};
        }
        return cat44(ds_lo, ds_hi);
    };

    // dQ^T += K^T (scale dS)^T over slots 32 h .. +31, K^T operands DA column
    // tiles ahead; step(mc) runs after each column tile's MFMA
    auto dq_loop = [&](auto H, bf16x8 dsb, auto&& step) {
        constexpr int h = decltype(H)::value;
        constexpr int DA = 4;
        bf16x8 kt[DA + 1];
#pragma unroll
        for (int k = 0; k < DA; ++k) kt[k] = Tile::slot_op(tile, TL, 32 * h, k);
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            if (mc + DA < MC) kt[(mc + DA) % (DA + 1)] = Tile::slot_op(tile, TL, 32 * h, mc + DA);
            acc[mc] = mfma16(kt[mc % (DA + 1)], dsb, acc[mc]);
            step(mc);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    s_loop(H0{}, [&](int ks) { gs.step(ks); });
    flags(H0{});
    s_loop(H1{}, [&](int ks) {
        if (ks < 8) epi_step(H0{}, ks);
    });
    const bf16x8 dsb0 = finish(H0{});
    flags(H1{});
    dq_loop(H0{}, dsb0, [&](int mc) {
        if (mc < 8) epi_step(H1{}, mc);
    });
    const bf16x8 dsb1 = finish(H1{});
    dq_loop(H1{}, dsb1, [](int) {});
}

template <int DQK>
__global__ __launch_bounds__(256, 1) void bwd_sdq_kernel(BwdArgs a) {
    using Tile = KvTileSwz<DQK>;
    constexpr int NW = 4, KS = DQK / 32, MC = DQK / 16, HT = NW * 16;
    __shared__ __attribute__((aligned(16))) __bf16 s_tile0[Tile::ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 s_tile1[Tile::ELEMS];
    __shared__ int s_rows[3][BLK];
    __shared__ int s_live[3];
    __shared__ int s_last[NW];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, n = lane & 15;
    // workgroup x -> (token, head group): the head groups of a token are 8
    // workgroups apart, so that they run on one XCD (workgroups go to the 8
    // XCDs in turn) at about the same time and the second gathers its rows
    // from that XCD's L2; tokens the chunk's longest rows first
    const int ngrp = (a.H + HT - 1) / HT;
    const int blk = (int)blockIdx.x / (8 * ngrp), rem = (int)blockIdx.x % (8 * ngrp);
    const int ti = blk * 8 + rem % 8;
    if (ti >= a.Tc) return;                            // uniform: past the chunk's tokens
    const int t = a.t0 + a.Tc - 1 - ti;
    const int h_wave = (rem / 8) * HT + wave * 16;
    const int head = h_wave + n;
    const bool hv = head < a.H;
    const bool active = h_wave < a.H;
    const int L = row_length(a.len, t, a.W);
    const int nblk = (L + BLK - 1) / BLK;

    f32x4 acc[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) acc[mc] = zero4();

    if (nblk == 0) {
        // an empty row: dQ = 0 below; Delta = O dO still when it is formed here
        if (a.o != nullptr && active) {
            float unused[1];
            fused_delta<1>(a, t, h_wave, lane,
                           [&](int, int ks, size_t row) { return ld8(a.dO + row * 512 + 32 * ks + 8 * g); },
                           unused);
        }
    } else {
        // q, dO (and the LSE, Delta scalars) go to registers once the first
        // tile's gather is in flight; with o given, Delta = sum O dO is formed
        // from dO before q is loaded
        // The LSE, sink and Delta scalars load first; q and dO go out right
        // behind the row's first indices (early), so that the wait for those
        // indices does not wait for them; their arithmetic waits until the
        // first tile's gather is in flight (post).  With o given, Delta =
        // sum O dO is formed there from dO and O.  Lanes of heads past H load
        // head 0's row (the loads stay unconditional: the compiler loses
        // count of loads issued inside a branch and would then drain them at
        // the indices' wait) and zero it.
        bf16x8 qop[KS], dop[16];
        const size_t row = (size_t)t * a.H + (hv ? head : 0);
        const float l_raw = a.lse[row];
        const float sk_raw = a.sink ? a.sink[hv ? head : 0] : 0.f;
        float lse2 = 0.f, dlt = a.o == nullptr ? a.delta[row] : 0.f;
        auto early = [&]() {
#pragma unroll
            for (int ks = 0; ks < 16; ++ks) {
                const bf16x8 x = ld8(a.dO + row * 512 + 32 * ks + 8 * g);
                dop[ks] = hv ? x : zero8();
            }
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 x = ld8(a.q + row * DQK + 32 * ks + 8 * g);
                qop[ks] = hv ? x : zero8();
            }
        };
        auto post = [&]() {
            // +inf for a saturating sink: every P is 0
            lse2 = hv ? (a.sink ? glae(l_raw, sk_raw) : l_raw) * LOG2E : 0.f;
            if (!hv) dlt = 0.f;
            if (a.o != nullptr && active) {     // uniform
                float d1[1];
                fused_delta<1>(a, t, h_wave, lane, [&](int, int ks, size_t) { return dop[ks]; }, d1);
                dlt = d1[0];
            }
        };
        const typename Tile::Lane TL = Tile::lane_bases(lane);
        gathered_blocks<DQK, NW>(a, s_tile0, s_tile1, s_rows, s_live, s_last, t, nblk, block_range(a, L),
                                 wave, lane,
                                 [&](const __bf16* tile, const int* rows, int b, const auto& gs, bool live) {
                                     if (active && live)
                                         sdq_block<DQK>(a, tile, TL, rows, qop, dop, lse2, dlt, acc, t, head, b,
                                                        lane, gs);
                                     else
                                         gs.all();
                                 }, post, early);
    }

    if (!hv) return;
    if (a.nsplit > 1) {
        // this split's share of dQ, in fp32, for dq_reduce_kernel
        float* dp = a.dq_part + (((size_t)(t - a.t0) * a.nsplit + blockIdx.z) * a.H + head) * DQK + 4 * g;
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) *reinterpret_cast<f32x4*>(dp + 16 * mc) = acc[mc];
        return;
    }
    // bf16 dQ: column tiles in pairs, regrouped over g (transpose_pairs) so
    // that lane (g, n) writes columns 32 k + 8 g .. +7 of head n, 16 bytes
    static_assert(MC % 2 == 0, "dQ column tiles go out in pairs");
    __bf16* dqp = a.dq + ((size_t)t * a.H + head) * DQK + 8 * g;
#pragma unroll
    for (int k = 0; k < MC / 2; ++k) {
        const f32x4 lo = acc[2 * k], hi = acc[2 * k + 1];
        u32x2 x0 = __builtin_bit_cast(u32x2, cvt4(lo[0], lo[1], lo[2], lo[3]));
        u32x2 x1 = __builtin_bit_cast(u32x2, cvt4(hi[0], hi[1], hi[2], hi[3]));
        transpose_pairs(x0, x1);
        *reinterpret_cast<u32x4*>(dqp + 32 * k) = u32x4{x0[0], x0[1], x1[0], x1[1]};
    }
}

// ---------------------------------------------------------------------------
// bwd_dkv: per token and 64-slot block,
//   u[slot][c] = sum_h (scale dS)[h][slot] q[h][c] + P[h][slot] dO[h][c]
// computed as u^T = q^T (scale dS) + dO^T P, a contraction over heads (HK
// k-steps of 32 heads).  Eight waves (two per SIMD, so one wave's stores
// overlap the other's MFMAs) split the 16-column tiles of d_qk: four d_v
// tiles each (q dS + dO P), and for d_qk = 576 one of the four rope tiles
// (q dS only) for each of the first four waves.
// q and dO for those columns stay in registers with heads in-lane, staged once
// per token through LDS with asynchronous loads (two buffers in flight).  The
// P / dS tiles of the next block load asynchronously while the current block
// is computed.  Each lane ends up holding 4 consecutive columns of u for one
// slot and writes them as one 8-byte store (a 4-value block) into the
// slot's row of the partial buffer; slots that are not valid are skipped.
// The stores go through a buffer resource over the token's partial rows
// (a 32-bit lane offset, the block and quarter in the scalar offset): a
// 64-bit row pointer per lane would not fit the register budget, and a
// spilled one reloads with a wait on every outstanding load and store.
// ---------------------------------------------------------------------------

// P or scale*dS tile: [HP heads][64 slots] bf16, 128-byte rows, chunk c of row
// h stored at c ^ pf(h) so that the transposed reads (4 consecutive heads x 32
// bytes per 16 lanes, two lane groups 8 heads apart per 32 lanes) avoid bank
// conflicts.
__device__ __forceinline__ int pf(int h) { return (((h >> 1) & 1) << 1) | (((h >> 3) & 1) << 2); }

// Chunk permutation of the staged q / dO rows: stage_op reads rows
// {8g + i, 8g + 4 + i}, and each 32-lane pass of its transposed reads must
// see 8 rows on distinct banks (1152-byte rows alternate between two bank
// halves by themselves; 1024-byte rows all start at bank 0).
template <int D>
struct StageF;
template <>
struct StageF<576> {
    __device__ static int f(int r) { return (((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2); }
};
template <>
struct StageF<512> {
    __device__ static int f(int r) { return ((r & 3) << 1) | (((r >> 3) & 1) << 3); }
};

template <int D, int NW>
__device__ __forceinline__ void stage_rows_async(__bf16* dst, const __bf16* src_rows, int nrows_valid,
                                                 int wave_s, int lane) {
    // 32 rows x D columns; rows >= nrows_valid repeat the last valid row
    constexpr int CH = D / 8;
    constexpr int INSTR = 32 * CH / 64;
    int lv;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lv) : "v"(lane));
#pragma unroll
    for (int k = 0; k < (INSTR + NW - 1) / NW; ++k) {
        const int i = k * NW + wave_s;
        if (INSTR % NW != 0 && i >= INSTR) break;     // wave-uniform
        const int pos = i * 64 + lv;
        const int row = pos / CH;
        const int pc = pos - row * CH;
        const int rr = row < nrows_valid ? row : nrows_valid - 1;
        const __bf16* src = src_rows + (size_t)rr * D + ((pc ^ StageF<D>::f(row)) << 3);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_void*)(dst + i * 512), 16, 0, 0);
    }
}

// B-operand read of staged rows: lane (g, n) gets rows 8g..8g+7 (as two
// transposed 4-row reads) of column c0 + n.
template <int D>
__device__ __forceinline__ bf16x8 stage_op(const __bf16* stage, int c0, int lane) {
    const int g = lane >> 4, w = lane & 15;
    const int row = 8 * g + (w >> 2);
    const int col = c0 + 4 * (w & 3);
    const int e0 = row * D + ((((col >> 3) ^ StageF<D>::f(row))) << 3) + (col & 7);
    const int e1 = (row + 4) * D + ((((col >> 3) ^ StageF<D>::f(row + 4))) << 3) + (col & 7);
    return cat44(lds_tr4(stage + e0), lds_tr4(stage + e1));
}

// Issue the loads of the [P | scale dS] tiles of block b into buf (rows
// h < H of each; pieces of 8 head rows = 1 KB, a fixed number per wave so
// the loop unrolls and keeps no loop state in registers).  No wait here.
template <int HP, int NW>
__device__ __forceinline__ void pd_tiles_async(const BwdArgs& a, __bf16* buf, int t, int b,
                                               int wave_s, int lane) {
    constexpr int NP = HP / 8;                     // pieces per tile (8 head rows each)
    static_assert((2 * NP) % NW == 0, "pieces must split evenly over the waves");
    const int row_in = lane >> 3, pc = lane & 7;
#pragma unroll
    for (int k = 0; k < 2 * NP / NW; ++k) {
        const int i = k * NW + wave_s;
        const int which = i >= NP;                 // 0: P, 1: scale dS
        const int piece = i - which * NP;
        const int h = 8 * piece + row_in;
        if (h < a.H) {
            const __bf16* src = (which ? a.ws_ds : a.ws_p) + ((size_t)(t - a.t0) * a.H + h) * a.Wp + b * BLK +
                                ((pc ^ pf(h)) << 3);
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             (lds_void*)(buf + which * HP * BLK + 8 * piece * BLK), 16, 0, 0);
        }
    }
}

// B-operand read of a P / dS tile: lane (g, n) gets heads h0 + 8g .. +7 of
// slot s0 + n.
__device__ __forceinline__ bf16x8 pd_op(const __bf16* tile, int h0, int s0, int lane) {
    const int g = lane >> 4, w = lane & 15;
    const int h = h0 + 8 * g + (w >> 2);
    const int col = s0 + 4 * (w & 3);
    const int e0 = h * BLK + ((((col >> 3) ^ pf(h))) << 3) + (col & 7);
    const int e1 = (h + 4) * BLK + ((((col >> 3) ^ pf(h + 4))) << 3) + (col & 7);
    return cat44(lds_tr4(tile + e0), lds_tr4(tile + e1));
}

// The four 8-byte blocks that lanes (g, n), g = 0..3, hold for one slot n
// and column tile nt (columns c + 16 nt + 4 g .. +3), transposed over g: lane g
// ends with tile g's 32 contiguous bytes (its four blocks in column order), so
// a slot's 128 bytes go out as two 16-byte stores per lane instead of four
// 8-byte ones.  Two swap steps between 16-lane rows: rows 2, 3 of tiles 0, 1
// with rows 0, 1 of tiles 2, 3; then rows 1, 3 of tiles 0, 2 with rows 0, 2 of
// tiles 1, 3.
__device__ __forceinline__ void transpose_blocks(u32x2 (&r)[4]) {
#pragma unroll
    for (int d = 0; d < 2; ++d)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto x = __builtin_amdgcn_permlane32_swap(r[d][w], r[2 + d][w], false, false);
            r[d][w] = x[0];
            r[2 + d][w] = x[1];
        }
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto x = __builtin_amdgcn_permlane16_swap(r[2 * c][w], r[2 * c + 1][w], false, false);
            r[2 * c][w] = x[0];
            r[2 * c + 1][w] = x[1];
        }
}

template <int DQK, int HK, int MW, int RW, bool ROPE>
__device__ __forceinline__ void dkv_block(const BwdArgs& a, const __bf16* pd, const int* raw,
                                          const bf16x8 (&qB)[HK][MW + RW], const bf16x8 (&dB)[HK][MW], int b,
                                          int L, __amdgpu_buffer_rsrc_t prs, int voff, int voff_rope, int lane) {
    constexpr int HP = 32 * HK;
    const int n = lane & 15;
    {
        // a block without a valid slot writes nothing (and its P / dS tile
        // was never stored): skip it
        const int v = raw[lane];
        if (__builtin_amdgcn_ballot_w64(b * BLK + lane < L && v >= 0 && v < a.S_kv) == 0) return;
    }
    // four quarters of 16 slots: one accumulator tile per column tile
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
        f32x4 acc[MW + 1];
#pragma unroll
        for (int nt = 0; nt <= MW; ++nt) acc[nt] = zero4();
#pragma unroll
        for (int hk = 0; hk < HK; ++hk) {
            const bf16x8 bp = pd_op(pd, 32 * hk, 16 * qt, lane);
            const bf16x8 bds = pd_op(pd + HP * BLK, 32 * hk, 16 * qt, lane);
#pragma unroll
            for (int nt = 0; nt < MW; ++nt) {
                acc[nt] = mfma16(qB[hk][nt], bds, acc[nt]);
                acc[nt] = mfma16(dB[hk][nt], bp, acc[nt]);
            }
            // a rope column tile: q dS only (dO has no columns there)
            if constexpr (ROPE) acc[MW] = mfma16(qB[hk][MW], bds, acc[MW]);
        }
        // lane (g, n) holds columns c + 4g .. +3 of slot 16 qt + n for each of
        // its column tiles, one 4-value block (8 bytes) each; the main tiles'
        // blocks are transposed over g (all four lanes of a slot take part: a
        // slot's validity is the same for them) and stored 16 bytes at a time.
        // Only valid slots are written (the row lists name no other slot).
        u32x2 blk[MW];
#pragma unroll
        for (int nt = 0; nt < MW; ++nt) blk[nt] = pack_blk4(acc[nt]);
        transpose_blocks(blk);
        const int slot = 16 * qt + n;
        const int v = raw[slot];
        if (b * BLK + slot < L && v >= 0 && v < a.S_kv) {
            const int soff = 16 * qt * (2 * DQK);         // prs starts at the block's first slot row
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{blk[0][0], blk[0][1], blk[1][0], blk[1][1]}, prs, voff,
                                                   soff, 0);
            __builtin_amdgcn_raw_buffer_store_b128(u32x4{blk[2][0], blk[2][1], blk[3][0], blk[3][1]}, prs,
                                                   voff + 16, soff, 0);
            if constexpr (ROPE) __builtin_amdgcn_raw_buffer_store_b64(pack_blk4(acc[MW]), prs, voff_rope, soff, 0);
        }
    }
}

template <int DQK, int HK>
__global__ __launch_bounds__(512, 1) void bwd_dkv_kernel(BwdArgs a) {
    constexpr int DV = 512;
    constexpr int NW = 8;
    constexpr int MW = DV / 16 / NW;                    // main (d_v) column tiles per wave: 4
    constexpr int RW = (DQK - DV) / 16 > 0 ? 1 : 0;     // a rope column tile, for the first RN waves
    constexpr int RN = (DQK - DV) / 16;                 // rope column tiles (4 or 0)
    static_assert(RN <= NW, "one rope column tile per wave at most");
    constexpr int HP = 32 * HK;                         // heads padded
    // four LDS buffers of one size: all four take the staged q / dO pieces in
    // turn (three in flight); afterwards s_pd1 / s_pd0 hold the [P | dS] tiles
    // of even / odd blocks
    constexpr int SLOT = 32 * DQK > 2 * HP * BLK ? 32 * DQK : 2 * HP * BLK;
    __shared__ __attribute__((aligned(16))) __bf16 s_st0[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 s_st1[SLOT];
    __shared__ __attribute__((aligned(16))) __bf16 s_pd0[SLOT];   // [P | dS], even blocks
    __shared__ __attribute__((aligned(16))) __bf16 s_pd1[SLOT];   // [P | dS], odd blocks; staging
    __shared__ int s_raw[2][BLK];                                  // raw top-k indices

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t = a.t0 + a.Tc - 1 - (int)blockIdx.x;     // the chunk's longest rows first
    const int L = row_length(a.len, t, a.W);
    // the row's blocks [b_lo, b_end) (all of them without a split)
    const int nblk = (L + BLK - 1) / BLK;
    const int b_lo = a.nsplit > 1 ? (int)blockIdx.z * a.bps : 0;
    const int b_end = a.nsplit > 1 && b_lo + a.bps < nblk ? b_lo + a.bps : nblk;
    if (b_end <= b_lo) return;             // uniform: an empty row (or range) adds nothing
    // wave w owns main column tiles [MW w, MW w + MW) (columns 64 w ..) and,
    // for w < RN, rope column tile w (columns 512 + 16 w ..): every MFMA has
    // real operands, and the two waves of a SIMD issue 9 + 8 of them per
    // 32-head step
    const int c_wave = 16 * MW * wave;
    const bool has_rope = RW > 0 && wave < RN;           // uniform
    const int c_rope = DV + 16 * wave;

    // heads past H: their P / dS tile rows stay zero (never loaded; s_pd0 and
    // s_pd1 are cleared after their last turn as staging buffers)
    auto zero_rows_past_h = [&](__bf16* buf) {
        for (int i = a.H * BLK / 8 + tid; i < HP * BLK / 8; i += NW * 64) {
            reinterpret_cast<u32x4*>(buf)[i] = u32x4{0u, 0u, 0u, 0u};
            reinterpret_cast<u32x4*>(buf + HP * BLK)[i] = u32x4{0u, 0u, 0u, 0u};
        }
    };

    // ---- q and dO with heads in-lane: lane (g, n) of k-step hk, column tile
    // nt holds X[32hk + 8g + j][c + n], j = 0..7, c the tile's first column
    // (c_wave + 16 nt, or c_rope for the rope tile nt = MW).  Staged in 2*HK
    // pieces of 32 head rows (rows past H repeat row H-1: their P and dS are
    // zero) through a ring of all four buffers: pieces p + 1 .. p + 3 load
    // while piece p is read, about 110 KB in flight.  The [P | dS] tile of
    // block 0 loads into s_pd1 as soon as the ring is done with it; the blocks
    // then take s_pd1 (even) and s_pd0 (odd).
    bf16x8 qB[HK][MW + RW], dB[HK][MW];
    constexpr int NPC = 2 * HK;
    constexpr int RING = 4;
    // the last piece staged in s_pd1 (ring slot 2), -1 if none; never the
    // last piece (NPC is even)
    constexpr int LAST_PD1 = NPC > 2 ? ((NPC - 1 - 2) / RING) * RING + 2 : -1;
    static_assert(NPC % 2 == 0 && LAST_PD1 < NPC - 1, "s_pd1 is free before the last piece");
    __bf16* const ring[RING] = {s_st0, s_st1, s_pd1, s_pd0};
    auto issue = [&](int piece) {
        const int hk = piece >> 1;
        const int nv = a.H - 32 * hk;
        const size_t row0 = (size_t)t * a.H + 32 * hk;
        if ((piece & 1) == 0) stage_rows_async<DQK, NW>(ring[piece % RING], a.q + row0 * DQK, nv, wave, lane);
        else stage_rows_async<DV, NW>(ring[piece % RING], a.dO + row0 * DV, nv, wave, lane);
    };
    auto first_tile = [&]() {
        if (HP > a.H) zero_rows_past_h(s_pd1);
        pd_tiles_async<HP, NW>(a, s_pd1, t, b_lo, wave, lane);
    };
    // each wave issues at least 4 loads per piece (d_qk or d_v columns x 32
    // rows in 16-byte loads over 8 waves): with k pieces issued after piece p,
    // waiting down to 4 k outstanding loads completes every load of piece p
    // (loads complete in issue order)
    static_assert((32 * (DV / 8) / 64) / NW >= 4, "the ring waits assume at least 4 loads per piece");
    if (wave == 0) stage_slot_idx(s_raw[0], a.idx, t, a.W, b_lo, lane);
    if (LAST_PD1 < 0) first_tile();
#pragma unroll
    for (int piece = 0; piece < RING - 1 && piece < NPC; ++piece) issue(piece);
#pragma unroll
    for (int piece = 0; piece < NPC; ++piece) {
        // pieces piece + 1, piece + 2 stay in flight.  A plain barrier: the
        // workgroup fence of __syncthreads would wait for every outstanding
        // LDS-bound load.  lgkmcnt(0): this wave's reads of piece - 1 are
        // done before its buffer is reloaded.
        const int after = NPC - 1 - piece < RING - 2 ? NPC - 1 - piece : RING - 2;
        if (after == 2) asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else if (after == 1) asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        else asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (piece + RING - 1 < NPC) issue(piece + RING - 1);     // into the buffer of piece - 1
        if (LAST_PD1 >= 0 && piece == LAST_PD1 + 1) first_tile();   // s_pd1's last piece is read
        const __bf16* cur = ring[piece % RING];
        const int hk = piece >> 1;
        // operands are read unconditionally (column clamped into the piece)
        // and zeroed after: no branch around the LDS reads
#pragma unroll
        for (int nt = 0; nt < MW; ++nt) {
            const int c0 = c_wave + 16 * nt;
            if ((piece & 1) == 0) qB[hk][nt] = stage_op<DQK>(cur, c0, lane);
            else dB[hk][nt] = stage_op<DV>(cur, c0, lane);
        }
        // the rope tile's q (read by every wave, the column clamped into the
        // piece, and zeroed where the wave has none: no branch around the
        // LDS read)
        if (RW > 0 && (piece & 1) == 0) {
            const bf16x8 x = stage_op<DQK>(cur, RW > 0 && wave < RN ? c_rope : 0, lane);
            qB[hk][MW + RW - 1] = has_rope ? x : zero8();
        }
    }
    // s_pd0 (ring slot 3) is done after the last piece: every wave must have
    // read it before its padded rows are cleared; the block loop's first
    // barrier then orders the clearing before the reads.
    if (HP > a.H) {
        __syncthreads();
        zero_rows_past_h(s_pd0);
    }

    // ---- blocks: [P | dS] tiles double-buffered.  A block's partial rows
    // (64 rows of 2 d_qk bytes) through a buffer resource based at the
    // block's first row (64-bit address: a token's rows may span more than
    // 2^31 bytes): lane (g, n) stores slot 16 qt + n, columns c_wave + 16g ..
    // +15 (the main tiles, after the transpose) and c_rope + 4g .. +3 (its
    // rope tile)
    char* const part_t = reinterpret_cast<char*>(a.partial) + (size_t)(t - a.t0) * a.Wp * (2 * DQK);
    static_assert(MW == 4, "the block transpose takes four main column tiles per wave");
    const int voff = (lane & 15) * (2 * DQK) + 2 * (c_wave + 16 * (lane >> 4));
    const int voff_rope = (lane & 15) * (2 * DQK) + 2 * (c_rope + 4 * (lane >> 4));
    // one copy of the block per kind of wave, so the MFMAs stay in one basic block
    auto block = [&](const __bf16* pd, const int* raw, int b) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t prs = __builtin_amdgcn_make_buffer_rsrc(
            part_t + (size_t)b * (BLK * 2 * DQK), (short)0, BLK * 2 * DQK, 0x00020000);
        if (has_rope)
            dkv_block<DQK, HK, MW, RW, RW != 0>(a, pd, raw, qB, dB, b, L, prs, voff, voff_rope, lane);
        else
            dkv_block<DQK, HK, MW, RW, false>(a, pd, raw, qB, dB, b, L, prs, voff, voff_rope, lane);
    };
    for (int b = b_lo; b < b_end; b += 2) {
        wait_vmem();
        __syncthreads();
        if (b + 1 < b_end) {
            pd_tiles_async<HP, NW>(a, s_pd0, t, b + 1, wave, lane);
            if (wave == 0) stage_slot_idx(s_raw[1], a.idx, t, a.W, b + 1, lane);
        }
        block(s_pd1, s_raw[0], b);
        if (b + 1 >= b_end) break;
        wait_vmem();
        __syncthreads();
        if (b + 2 < b_end) {
            pd_tiles_async<HP, NW>(a, s_pd1, t, b + 2, wave, lane);
            if (wave == 0) stage_slot_idx(s_raw[0], a.idx, t, a.W, b + 2, lane);
        }
        block(s_pd0, s_raw[1], b + 1);
    }
}

// ---------------------------------------------------------------------------
// dKV reduce, two levels, fixed order (so dkv is the same bits every run):
//   dkv_part     one wave per part (<= RPART consecutive entries of one row's
//                list): sums the listed partial rows in list (token) order
//   dkv_combine  one wave per KV row: sums the row's parts in order and writes
//                dkv (rows that no valid slot names get 0)
// Cutting long lists into parts keeps every wave's work bounded: the first KV
// rows are named by thousands of tokens, the last ones by a few.
// Lane l owns columns 4l..4l+3 (+256, +512 as needed).
// ---------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(256) void dkv_part_kernel(BwdArgs a) {
    // lane l < DQK / 16 owns columns 16 l .. 16 l + 15: four 8-byte blocks,
    // two 16-byte loads per row
    constexpr int G = DQK / 16;
    constexpr int U = 4;                       // partial rows in flight per wave
    const int p = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (p >= a.part_off[a.S_kv]) return;
    const int r = a.part_row[p];
    const int lo = a.row_off[r] + (p - a.part_off[r]) * RPART;
    const int hi = lo + RPART < a.row_off[r + 1] ? lo + RPART : a.row_off[r + 1];
    const int cnt = hi - lo;                   // 1..RPART
    const int my_ent = lane < cnt ? a.entries[lo + lane] : 0;
    const bool act = lane < G;
    f32x4 acc[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) acc[v] = zero4();
    for (int k0 = 0; k0 < cnt; k0 += U) {
        u32x4 x[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int e = __shfl(my_ent, k0 + u, 64);
            const u32x4* src = reinterpret_cast<const u32x4*>(reinterpret_cast<const char*>(a.partial) +
                                                              (size_t)e * (2 * DQK) + 32 * lane);
#pragma unroll
            for (int v = 0; v < 2; ++v) x[u][v] = (k0 + u < cnt && act) ? src[v] : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[0] += unpack_blk4(u32x2{x[u][0][0], x[u][0][1]});
            acc[1] += unpack_blk4(u32x2{x[u][0][2], x[u][0][3]});
            acc[2] += unpack_blk4(u32x2{x[u][1][0], x[u][1][1]});
            acc[3] += unpack_blk4(u32x2{x[u][1][2], x[u][1][3]});
        }
    }
    if (act) {
#pragma unroll
        for (int v = 0; v < 4; ++v)
            *reinterpret_cast<f32x4*>(a.part_sum + (size_t)p * DQK + 16 * lane + 4 * v) = acc[v];
    }
}

template <int DQK>
__global__ __launch_bounds__(256) void dkv_combine_kernel(BwdArgs a) {
    constexpr int NV = (DQK / 4 + 63) / 64;
    const int r = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (r >= a.S_kv) return;
    const int p0 = a.part_off[r], p1 = a.part_off[r + 1];
    // the first chunk writes every row (0 where no slot of it names the row);
    // a later chunk adds its sum to the rows it names, so a row's total is
    // summed chunk by chunk in token order
    const bool first = a.t0 == 0;
    if (!first && p0 == p1) return;
    f32x4 acc[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) acc[v] = zero4();
    // four parts' loads in flight, summed in part order (the first rows have
    // tens of parts: a load round trip per part would set the kernel's time)
    constexpr int UP = 4;
    int p = p0;
    for (; p + UP <= p1; p += UP) {
        f32x4 x[UP][NV];
#pragma unroll
        for (int k = 0; k < UP; ++k)
#pragma unroll
            for (int v = 0; v < NV; ++v) {
                const int c = 4 * (lane + 64 * v);
                x[k][v] = c < DQK ? *reinterpret_cast<const f32x4*>(a.part_sum + (size_t)(p + k) * DQK + c) : zero4();
            }
#pragma unroll
        for (int k = 0; k < UP; ++k)
#pragma unroll
            for (int v = 0; v < NV; ++v) acc[v] += x[k][v];
    }
    for (; p < p1; ++p) {
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const int c = 4 * (lane + 64 * v);
            if (c < DQK) acc[v] += *reinterpret_cast<const f32x4*>(a.part_sum + (size_t)p * DQK + c);
        }
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const int c = 4 * (lane + 64 * v);
        if (c < DQK) {
            f32x4* dst = reinterpret_cast<f32x4*>(a.dkv + (size_t)r * DQK + c);
            *dst = first ? acc[v] : *dst + acc[v];
        }
    }
}

// ---------------------------------------------------------------------------
// d_sink[h] = -sum_t p_sink[t,h] * delta[t,h], p_sink = sigmoid(sink - lse);
// empty rows (lse = -inf) are skipped; one workgroup per head, fixed order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void dsink_kernel(const float* __restrict__ lse,
                                                    const float* __restrict__ delta,
                                                    const float* __restrict__ sink,
                                                    float* __restrict__ d_sink, int T, int H) {
    __shared__ float s_part[256];
    const int h = blockIdx.x;
    const float sk = sink[h];
    float acc = 0.f;
    // U tokens per thread in flight (the loads of a head are H floats apart,
    // one 64-byte segment each: latency, not bandwidth, sets the time)
    constexpr int U = 8;
    for (int t0 = threadIdx.x; t0 < T; t0 += 256 * U) {
        float l[U], d[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = t0 + 256 * u;
            l[u] = t < T ? lse[(size_t)t * H + h] : -INFINITY;
            d[u] = t < T ? delta[(size_t)t * H + h] : 0.f;
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (l[u] == -INFINITY) continue;
            float ps;
            if (sk == -INFINITY) ps = 0.f;
            else if (sk == INFINITY && l[u] == INFINITY) ps = 0.5f;
            else ps = sigmoid(sk - l[u]);
            acc += ps * d[u];
        }
    }
    s_part[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) s_part[threadIdx.x] += s_part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) d_sink[h] = -s_part[0];
}

// stage boundaries: 0 start | 1 index inversion | 2 S/dP and dQ | 3 dQ merge
// (split block ranges) | 4 dkv | 5 reduce | 6 d_sink.  With several token chunks, events 1-5 are recorded
// during the first chunk only (they bracket its stages) and event 6 after the
// whole call.
struct Marks {
    hipEvent_t* ev;
    hipStream_t stream;
    hipError_t* err;
    bool on;
    __host__ void operator()(int i) const {
        if (ev == nullptr || !on) return;
        const hipError_t e = hipEventRecord(ev[i], stream);
        if (*err == hipSuccess) *err = e;
    }
};

// The index inversion of the chunk in a (rows of every range, token order).
static hipError_t launch_inversion(const BwdArgs& a, hipStream_t stream) {
    const int nr = a.S_kv < INV_ROWS ? a.S_kv : INV_ROWS;
    const size_t lds = (size_t)nr * sizeof(int);
    if (a.S_kv <= INV_ROWS && a.W <= SMALL_INV_W && a.Tc <= SMALL_INV_TOKENS) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(rows_small_kernel),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        hipLaunchKernelGGL(rows_small_kernel, dim3(1), dim3(1024), lds, stream, a);
        return hipSuccess;
    }
    hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(rows_count_kernel),
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err == hipSuccess)
        err = hipFuncSetAttribute(reinterpret_cast<const void*>(rows_fill_kernel),
                                  hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
    const dim3 grid(a.nsub, (a.S_kv + INV_ROWS - 1) / INV_ROWS);
    hipLaunchKernelGGL(rows_count_kernel, grid, dim3(256), lds, stream, a);
    hipLaunchKernelGGL(rows_chunkscan_kernel, dim3((a.S_kv + 31) / 32), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(rows_scan_kernel, dim3(1), dim3(1024), 0, stream, a);
    hipLaunchKernelGGL(rows_parts_kernel, dim3((a.S_kv + 255) / 256), dim3(256), 0, stream, a);
    hipLaunchKernelGGL(rows_fill_kernel, grid, dim3(256), lds, stream, a);
    return hipSuccess;
}

template <int DQK, int HK>
static void launch_dkv_t(const BwdArgs& a, hipStream_t stream) {
    hipLaunchKernelGGL((bwd_dkv_kernel<DQK, HK>), dim3(a.Tc, 1, a.nsplit > 1 ? a.nsplit : 1), dim3(512), 0,
                       stream, a);
}

// One token chunk: inversion, S/P/dP/dS, dQ, dKV partials, reduce into dkv.
template <int DQK>
static hipError_t launch_chunk_t(const BwdArgs& a, hipStream_t stream, const Marks& mark) {
    const hipError_t err = launch_inversion(a, stream);
    if (err != hipSuccess) return err;
    mark(1);
    const int hk = (a.H + 31) / 32;
    const int ns = a.nsplit > 1 ? a.nsplit : 1;    // workgroups per token (block ranges)
    // S/dP and dQ: one workgroup per token and group of 64 heads (4 waves of
    // 16, one per SIMD: q, dO and the dQ^T accumulators take most of the
    // register file); a token's groups are numbered 8 apart, so they run on
    // one XCD and the second finds the gathered rows in its L2.
    hipLaunchKernelGGL((bwd_sdq_kernel<DQK>), dim3((a.Tc + 7) / 8 * 8 * ((a.H + 63) / 64), 1, ns), dim3(256), 0,
                       stream, a);
    mark(2);
    if (ns > 1)
        hipLaunchKernelGGL((dq_reduce_kernel<DQK>), dim3((a.Tc * a.H + 3) / 4), dim3(256), 0, stream, a);
    mark(3);
    switch (hk) {
        case 1: launch_dkv_t<DQK, 1>(a, stream); break;
        case 2: launch_dkv_t<DQK, 2>(a, stream); break;
        case 3: launch_dkv_t<DQK, 3>(a, stream); break;
        default: launch_dkv_t<DQK, 4>(a, stream); break;
    }
    mark(4);
    hipLaunchKernelGGL((dkv_part_kernel<DQK>), dim3((a.max_parts + 3) / 4), dim3(256), 0, stream, a);
    hipLaunchKernelGGL((dkv_combine_kernel<DQK>), dim3((a.S_kv + 3) / 4), dim3(256), 0, stream, a);
    mark(5);
    return hipSuccess;
}

// Exact Delta: the S / dP half of bwd_sdq, accumulating sum_j P_j dP_j
// instead of storing P and dS.
template <int DQK>
static void launch_delta_exact_t(const BwdArgs& a, hipStream_t stream) {
    // a.t0 = 0, a.Tc = T: every token
    if (a.H > 64)
        hipLaunchKernelGGL((delta_exact_kernel<DQK, 8, 1>), dim3(a.T, 1), dim3(512), 0, stream, a);
    else
        hipLaunchKernelGGL((delta_exact_kernel<DQK, 4, 1>), dim3(a.T, 1), dim3(256), 0, stream, a);
}

hipError_t launch_delta_exact(int d_qk, const BwdArgs& a, hipStream_t stream) {
    if (d_qk == 576) launch_delta_exact_t<576>(a, stream);
    else launch_delta_exact_t<512>(a, stream);
    return hipGetLastError();
}

hipError_t launch_bwd(int d_qk, const BwdArgs& args, float* d_sink, hipStream_t stream,
                      hipEvent_t* ev) {
    hipError_t err = hipSuccess;
    Marks mark{ev, stream, &err, true};
    mark(0);
    if (args.T > 0) {
        // token chunks of args.Tc tokens (the last one may be shorter), in
        // token order: the workspace holds one chunk
        for (int t0 = 0; t0 < args.T && err == hipSuccess; t0 += args.Tc) {
            BwdArgs a = args;
            a.t0 = t0;
            a.Tc = args.T - t0 < args.Tc ? args.T - t0 : args.Tc;
            a.tchunk = (a.Tc + a.nsub - 1) / a.nsub;
            a.nsub = (a.Tc + a.tchunk - 1) / a.tchunk;
            mark.on = t0 == 0;
            const hipError_t e = d_qk == 576 ? launch_chunk_t<576>(a, stream, mark)
                                             : launch_chunk_t<512>(a, stream, mark);
            if (err == hipSuccess) err = e;
        }
        mark.on = true;
    } else {
        // no tokens: dkv is all zeros
        mark(1);
        const size_t n = (size_t)args.S_kv * d_qk;
        const size_t want = (n + 255) / 256;
        const int fb = (int)(want < 4096 ? want : 4096);
        hipLaunchKernelGGL(fill_i32_kernel, dim3(fb), dim3(256), 0, stream,
                           reinterpret_cast<int*>(args.dkv), 0, n);
        mark(2); mark(3); mark(4); mark(5);
    }
    if (args.sink != nullptr)
        hipLaunchKernelGGL(dsink_kernel, dim3(args.H), dim3(256), 0, stream, args.lse, args.delta, args.sink,
                           d_sink, args.T, args.H);
    mark(6);
    const hipError_t le = hipGetLastError();
    return le != hipSuccess ? le : err;
}

}  // namespace smla
