// Sparse MLA forward for gfx950: one workgroup per (token, head tile).
//
// Method ([flash-attn #2882] Agent Notes; [cuDNN-FE #785] Summary 2-3): for
// each token, the H query heads share the token's gathered KV rows.  Per block
// of 64 top-k slots the workgroup
//   0. (once) finds the row's last valid slot: the blocks after its block
//      hold only padding (the tail of a non-compact row) and are not run,
//      as a compact row's length bounds its block count ([cuDNN-FE #785]
//      Summary 2); a block without a valid slot adds exact zeros everywhere,
//      so the output is the same bits;
//   1. resolves slot -> KV row (invalid slots -> -1) two blocks ahead;
//   2. gathers the rows of the NEXT block into the other of two LDS tiles with
//      asynchronous direct global->LDS 16-byte loads, so that the gather of
//      block b+1 is in flight while block b is computed (the pages find the
//      gather latency to be the bottleneck, [flash-attn #2882] Performance).
//      The loads are issued one per k-step of the first half's S^T loop: the
//      address unit takes a 1 KB row load in about 20 cycles, so issuing a
//      wave's 18 loads back to back stalls it, while spread between MFMAs
//      they cost almost nothing;
//   3. computes S^T = K Q^T with bf16 MFMA (slots x heads, fp32 accumulate);
//      each wave owns NT x 16 heads and keeps their Q in registers; padded
//      heads (h >= H) are zero rows, so any H in 1..128 runs without padded
//      copies in memory ([flash-attn #2882] Mechanism);
//   4. masks invalid slots to -inf before any exponential ([cuDNN-FE #785]
//      Summary 2) and exponentiates in the log2 domain against a per-head
//      reference max fixed at the head's first valid block (no rescaling of
//      O inside the loop; see REF_SLACK);
//   5. accumulates O^T += V^T P^T, V^T read transposed from the same tile.
// The epilogue folds the sink, O = acc / l * sigmoid(lse - sink), the
// sink-free share of the softmax mass written without forming inf - inf
// ([cuDNN-FE #785] Why 3), stages O through LDS for coalesced stores, and
// writes the sink-free natural-log LSE.  Empty rows give O = 0, LSE = -inf.
#include "kv_tile.h"
#include "launch.h"

#include <type_traits>

namespace smla {

// A head's reference max is fixed at its first valid block and O is never
// rescaled inside the loop: P = 2^(s - m_ref) and the fp32 accumulators share
// fp32's exponent range, so scores up to REF_SLACK above the reference are
// exact up to rounding.  A token whose scores rise further than that is rerun
// with the exact max as reference (a second pass; rare).
constexpr float REF_SLACK = 64.0f;   // log2 units

template <int DQK, int NW, int NT>
struct FwdCfg {
    static constexpr int DV = 512;
    static constexpr int KS = DQK / 32;      // k-steps of S^T
    static constexpr int MC = DV / 16;       // 16-column tiles of O^T
    static constexpr int HT = NW * NT * 16;  // heads per workgroup
    using Tile = KvTileSwz<DQK>;
};

// One 64-slot block, as two halves of 32 slots: S^T for the half, mask,
// P = 2^(s - m_ref), then O^T += V^T P^T over the half.
template <int DQK, int NW, int NT>
__device__ __forceinline__ void fwd_block(const FwdArgs& a, const __bf16* tile,
                                          const typename KvTileSwz<DQK>::Lane& TL, const int* rows,
                                          const bf16x8 (&qop)[NT][DQK / 32],
                                          f32x4 (&oacc)[512 / 16][NT], float (&m_ref)[NT],
                                          float (&rmax)[NT], float (&l_run)[NT],
                                          float (&l_rnd)[NT], int lane, __bf16* gtile,
                                          const int* grows, bool gnext, int wave) {
    using C = FwdCfg<DQK, NW, NT>;
    using Tile = typename C::Tile;
    const int g = lane >> 4;
    static_assert(NW == 4, "the gather schedule assumes 16 main rows and 2 rope loads per wave");
    const int gids = Tile::template row_ids<NW>(grows, wave, lane, a.S_kv);
    // the next block's gather reads nothing when there is no next block
    const auto kvr = Tile::kv_rsrc_if(a.kv, a.S_kv, gnext);

    // The block's two halves in the order S(0), S(1), PV(0), PV(1): the
    // exponentials of half 0 run between the MFMAs of S(1) and those of half
    // 1 between the MFMAs of PV(0), so the softmax's VALU work overlaps the
    // matrix work instead of leaving the MFMA pipe idle.  Each half's
    // arithmetic and its order are unchanged.
    f32x4 sacc[2][2][NT];                       // [half][m][nt]
    bf16x8 pop[2][NT];
    float psum[2][NT], m_use[2][NT];

    // S^T for slots 32 h .. +31 (K operands two k-steps ahead); step(ks)
    // runs after each k-step's MFMAs
    auto s_loop = [&](auto H, auto&& step) {
        constexpr int h = decltype(H)::value;
#pragma unroll
        for (int m = 0; m < 2; ++m)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sacc[h][m][nt] = zero4();
        constexpr int KD = 3;
        bf16x8 kop[KD][2];
#pragma unroll
        for (int i = 0; i < KD - 1; ++i)
#pragma unroll
            for (int m = 0; m < 2; ++m) kop[i][m] = Tile::row_op(tile, TL, (2 * h + m) * 16, i);
#pragma unroll
        for (int ks = 0; ks < C::KS; ++ks) {
            const int cur = ks % KD;
            if (ks + KD - 1 < C::KS) {
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    kop[(ks + KD - 1) % KD][m] = Tile::row_op(tile, TL, (2 * h + m) * 16, ks + KD - 1);
            }
#pragma unroll
            for (int m = 0; m < 2; ++m)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    sacc[h][m][nt] = mfma16(kop[cur][m], qop[nt][ks], sacc[h][m][nt]);
            step(ks);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // mask invalid slots before the exponential; log2-domain scores; the
    // reference max of heads that have none yet (all lanes of a head agree
    // after the reduction)
    auto prep = [&](auto H) {
        constexpr int h = decltype(H)::value;
        float hmax[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) hmax[nt] = -INFINITY;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = rows[(2 * h + m) * 16 + 4 * g + i] >= 0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float sv = ok ? sacc[h][m][nt][i] * a.scale_log2 : -INFINITY;
                    sacc[h][m][nt][i] = sv;
                    hmax[nt] = fmaxf(hmax[nt], sv);
                }
            }
        }
        bool unset = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            rmax[nt] = fmaxf(rmax[nt], hmax[nt]);
            unset |= m_ref[nt] == -INFINITY;
        }
        if (__builtin_amdgcn_ballot_w64(unset) != 0) {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float hm = xor_max(xor_max(hmax[nt], 16), 32);
                if (m_ref[nt] == -INFINITY) m_ref[nt] = hm;
            }
        }
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            m_use[h][nt] = (m_ref[nt] == -INFINITY) ? 0.f : m_ref[nt];
            psum[h][nt] = 0.f;
        }
    };

    // P = 2^(s - m_ref) for value k (0..7) of every head tile of half h
    auto exp_step = [&](auto H, int k) {
        constexpr int h = decltype(H)::value;
        const int m = k >> 2, i = k & 3;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const float p = fast_exp2(sacc[h][m][nt][i] - m_use[h][nt]);
            sacc[h][m][nt][i] = p;
            psum[h][nt] += p;
        }
    };

    // bf16 P as the B operand; the running sums
    auto finish = [&](auto H) {
        constexpr int h = decltype(H)::value;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            l_run[nt] += psum[h][nt];
            pop[h][nt] = cvt8(sacc[h][0][nt], sacc[h][1][nt]);
            // the sum of the bf16 weights the MFMA actually uses: O is
            // normalised by it, so O stays an exact convex combination of the
            // gathered V rows (a near one-hot row reproduces its V row)
            const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
            float rsum = l_rnd[nt];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                rsum = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{pop[h][nt][2 * j], pop[h][nt][2 * j + 1]}, one,
                                                       rsum, false);
            l_rnd[nt] = rsum;
        }
    };

    // O^T += V^T P^T over slots 32 h .. +31, V^T three column tiles ahead;
    // step(mc) runs after each column tile's MFMAs
    auto pv_loop = [&](auto H, auto&& step) {
        constexpr int h = decltype(H)::value;
        constexpr int VD = 4;
        bf16x8 vop[VD];
#pragma unroll
        for (int i = 0; i < VD - 1; ++i) vop[i] = Tile::slot_op(tile, TL, 32 * h, i);
#pragma unroll
        for (int mc = 0; mc < C::MC; ++mc) {
            const int cur = mc % VD;
            if (mc + VD - 1 < C::MC) vop[(mc + VD - 1) % VD] = Tile::slot_op(tile, TL, 32 * h, mc + VD - 1);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[mc][nt] = mfma16(vop[cur], pop[h][nt], oacc[mc][nt]);
            step(mc);
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    using H0 = std::integral_constant<int, 0>;
    using H1 = std::integral_constant<int, 1>;
    // S(0), issuing the next block's gather: one main row per k-step, then
    // the rope rows
    s_loop(H0{}, [&](int ks) {
        if (ks < 16) Tile::template gather_main_row<NW>(gtile, gids, kvr, wave, lane, ks);
        else Tile::template gather_rope_one<NW>(gtile, grows, kvr, wave, lane, ks - 16, a.S_kv);
    });
    prep(H0{});
    s_loop(H1{}, [&](int ks) {
        if (ks < 8) exp_step(H0{}, ks);
    });
    finish(H0{});
    prep(H1{});
    pv_loop(H0{}, [&](int mc) {
        if (mc < 8) exp_step(H1{}, mc);
    });
    finish(H1{});
    pv_loop(H1{}, [](int) {});
}

// topk_idxs[t][j] for any j (clamped into the row so the read is in bounds);
// its validity is decided later by valid_row, where the value is consumed.
__device__ __forceinline__ int raw_index(const FwdArgs& a, int t, int j) {
    return a.idx[(size_t)t * a.W + (j < a.W ? j : a.W - 1)];
}

__device__ __forceinline__ int valid_row(int v, int j, int L, int S_kv) {
    return (j < L && v >= 0 && v < S_kv) ? v : -1;
}

// SPLIT: the workgroup runs the blocks [b_lo, b_lo + bps) of split blockIdx.z
// only and writes its unnormalised O^T and softmax sums to the partials
// (merged by fwd_combine_kernel) instead of O and LSE.
template <int DQK, int NW, int NT, bool SPLIT>
__global__ __launch_bounds__(NW * 64, 1) void fwd_kernel(FwdArgs a) {
    using C = FwdCfg<DQK, NW, NT>;
    using Tile = typename C::Tile;
    constexpr int NTH = NW * 64;
    __shared__ __attribute__((aligned(16))) __bf16 s_tile0[Tile::ELEMS];
    __shared__ __attribute__((aligned(16))) __bf16 s_tile1[Tile::ELEMS];
    __shared__ int s_rows[3][BLK];
    __shared__ int s_last[NW];
    __shared__ int s_rerun;
    static_assert(64 * C::DV <= Tile::ELEMS && C::HT <= 128, "O staging must fit in the tiles");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // scalar
    const int g = lane >> 4, n = lane & 15;
    const int t = a.T - 1 - (int)blockIdx.x;          // longest rows first
    const int h_wg = (int)blockIdx.y * C::HT;
    const int h_wave = h_wg + wave * NT * 16;
    const bool active = h_wave < a.H;                 // wave-uniform
    const int L = row_length(a.len, t, a.W);
    const int split = SPLIT ? (int)blockIdx.z : 0;
    const int b_lo = SPLIT ? split * a.bps : 0;       // first block of this workgroup
    // slots this workgroup may run: [b_lo * BLK, j_hi)
    const int j_hi = SPLIT ? min(L, (b_lo + a.bps) * BLK) : L;

    if (tid == 0) s_rerun = 0;

    // Q as the B operand of S^T = K Q^T: lane (g, n) holds q[t, head, 32ks+8g..+7].
    // Loaded right behind the row's first indices (below), so that the wait
    // for those indices does not wait for q; unconditional loads (lanes of
    // heads past H read head 0's row and zero it), since the compiler loses
    // count of loads issued inside a branch and would drain them at that wait.
    bf16x8 qop[NT][C::KS];
    auto load_q = [&]() {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int head = h_wave + nt * 16 + n;
            const bool hv = head < a.H && L > 0;
            const __bf16* qp = a.q + ((size_t)t * a.H + (hv ? head : 0)) * DQK + 8 * g;
#pragma unroll
            for (int ks = 0; ks < C::KS; ++ks) {
                const bf16x8 x = ld8(qp + 32 * ks);
                qop[nt][ks] = hv ? x : zero8();
            }
        }
    };
    const typename Tile::Lane TL = Tile::lane_bases(lane);
    const auto kvr = Tile::kv_rsrc(a.kv, a.S_kv);
    f32x4 oacc[C::MC][NT];
    float m_ref[NT], rmax[NT], l_run[NT], l_rnd[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) m_ref[nt] = -INFINITY;

    // The row's last valid slot: the blocks after its block hold padding only
    // (the tail of a non-compact row), so the block loop ends there.  Each
    // wave's maximum goes to s_last, read after the first barrier below.  The
    // raw indices of the range's first 4 x NW x 64 slots and of its second
    // block load in one batch, q behind them: the slot rows of the first
    // block are v[0] of threads 0..63, those of the second block row1.
    static_assert(NTH >= 2 * BLK, "the first index batch must cover two blocks");
    int row0, row1;
    {
        const int j_first = b_lo * BLK;
        int v[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) v[k] = raw_index(a, t, j_first + k * NTH + tid);
        row1 = raw_index(a, t, j_first + BLK + (tid & (BLK - 1)));
        __builtin_amdgcn_sched_barrier(0);
        load_q();
        __builtin_amdgcn_sched_barrier(0);
        int last = -1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int j = j_first + k * NTH + tid;
            if (valid_row(v[k], j, j_hi, a.S_kv) >= 0) last = j;
        }
        for (int j0 = j_first + 4 * NTH; j0 < j_hi; j0 += 4 * NTH) {     // rows longer than one batch
            int u[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) u[k] = raw_index(a, t, j0 + k * NTH + tid);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int j = j0 + k * NTH + tid;
                if (valid_row(u[k], j, j_hi, a.S_kv) >= 0) last = j;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) last = max(last, __shfl_xor(last, m, 64));
        if (lane == 0) s_last[wave] = last;
        row0 = valid_row(v[0], j_first + (tid & (BLK - 1)), j_hi, a.S_kv);
        row1 = valid_row(row1, j_first + BLK + (tid & (BLK - 1)), j_hi, a.S_kv);
    }
    int nblk = 0;

    for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
        for (int mc = 0; mc < C::MC; ++mc)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) oacc[mc][nt] = zero4();
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) { rmax[nt] = -INFINITY; l_run[nt] = 0.f; l_rnd[nt] = 0.f; }

        if (tid < BLK) {
            s_rows[0][tid] = row0;
            s_rows[1][tid] = row1;
            s_rows[2][tid] = -1;     // written again before any block reads it
        }
        __syncthreads();
        if (pass == 0) {
            int last = s_last[0];
#pragma unroll
            for (int w = 1; w < NW; ++w) last = max(last, s_last[w]);
            nblk = __builtin_amdgcn_readfirstlane(last < 0 ? 0 : last / BLK + 1 - b_lo);
        }
        if (nblk > 0) Tile::template gather_async<NW>(s_tile0, s_rows[0], kvr, wave, lane, a.S_kv);

        // Two blocks per iteration so that each tile is a distinct LDS object.
        // Block k: wait for its tile; store the slot rows of block k + 1
        // (their raw indices were loaded at block k - 1 and the wait just
        // covered that load: storing them any earlier would wait for the whole
        // gather issued since); load the raw indices of block k + 2; compute,
        // issuing the gather of block k + 1 from inside the math (the last
        // block issues none).
        int ahead = 0;
        for (int b = 0; b < nblk; b += 2) {
            // ---- block b in tile 0
            wait_vmem();
            if (b > 0 && b + 1 < nblk && tid < BLK)
                s_rows[(b + 1) % 3][tid] = valid_row(ahead, (b_lo + b + 1) * BLK + tid, j_hi, a.S_kv);
            __syncthreads();
            ahead = tid < BLK ? raw_index(a, t, (b_lo + b + 2) * BLK + tid) : 0;
            __builtin_amdgcn_sched_barrier(0);
            if (active)
                fwd_block<DQK, NW, NT>(a, s_tile0, TL, s_rows[b % 3], qop, oacc, m_ref, rmax, l_run, l_rnd, lane,
                                       s_tile1, s_rows[(b + 1) % 3], b + 1 < nblk, wave);
            else if (b + 1 < nblk)
                Tile::template gather_async<NW>(s_tile1, s_rows[(b + 1) % 3], kvr, wave, lane, a.S_kv);
            if (b + 1 >= nblk) break;
            // ---- block b+1 in tile 1
            wait_vmem();
            if (b + 2 < nblk && tid < BLK)
                s_rows[(b + 2) % 3][tid] = valid_row(ahead, (b_lo + b + 2) * BLK + tid, j_hi, a.S_kv);
            __syncthreads();
            ahead = tid < BLK ? raw_index(a, t, (b_lo + b + 3) * BLK + tid) : 0;
            __builtin_amdgcn_sched_barrier(0);
            if (active)
                fwd_block<DQK, NW, NT>(a, s_tile1, TL, s_rows[(b + 1) % 3], qop, oacc, m_ref, rmax, l_run, l_rnd,
                                       lane, s_tile0, s_rows[(b + 2) % 3], b + 2 < nblk, wave);
            else if (b + 2 < nblk)
                Tile::template gather_async<NW>(s_tile0, s_rows[(b + 2) % 3], kvr, wave, lane, a.S_kv);
        }

        // did any head's scores rise more than REF_SLACK above its reference?
        bool far = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            rmax[nt] = xor_max(xor_max(rmax[nt], 16), 32);
            far |= rmax[nt] > m_ref[nt] + REF_SLACK;
        }
        if (pass == 0 && active && __builtin_amdgcn_ballot_w64(far) != 0 && lane == 0) s_rerun = 1;
        wait_vmem();
        __syncthreads();                // tiles and s_rows are free; s_rerun is final
        if (pass == 1 || s_rerun == 0) break;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) m_ref[nt] = rmax[nt];    // exact max: P <= 1
        __syncthreads();
    }

    if constexpr (SPLIT) {
        // partials of this split: the unnormalised O^T (lane (g, n) holds
        // columns 16 mc + 4g .. +3 of head n), and per head the reference
        // max (log2 domain; -inf without a valid slot), the fp32 sum of the
        // weights and the sum of their bf16 roundings.  Lane indices from an
        // opaque copy of the lane, as in the epilogue below.
        int lane_s;
        asm volatile("v_mov_b32 %0, %1" : "=v"(lane_s) : "v"(lane));
        const int g = lane_s >> 4, n = lane_s & 15;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int head = h_wave + nt * 16 + n;
            float l = l_run[nt], lr = l_rnd[nt];
            l += __shfl_xor(l, 16, 64);
            l += __shfl_xor(l, 32, 64);
            lr += __shfl_xor(lr, 16, 64);
            lr += __shfl_xor(lr, 32, 64);
            if (!active || head >= a.H) continue;
            const size_t row = ((size_t)t * a.nsplit + split) * a.H + head;
            float* op = a.opart + row * C::DV + 4 * g;
#pragma unroll
            for (int mc = 0; mc < C::MC; ++mc) *reinterpret_cast<f32x4*>(op + 16 * mc) = oacc[mc][nt];
            if (g == 0) *reinterpret_cast<f32x4*>(a.spart + row * 4) = f32x4{m_ref[nt], l, lr, 0.f};
        }
        return;
    }

    // epilogue: normalise, fold the sink, stage O^T through LDS as O rows.
    // The lane's indices are derived again from an opaque copy of the lane,
    // so that no epilogue address is computed ahead and kept live (and
    // spilled) across the block loop.
    int lane_e;
    asm volatile("v_mov_b32 %0, %1" : "=v"(lane_e) : "v"(lane));
    const int g_e = lane_e >> 4, n_e = lane_e & 15;
    float lse_v[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int head = h_wave + nt * 16 + n_e;
        float l = l_run[nt], lr = l_rnd[nt];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        lr += __shfl_xor(lr, 16, 64);
        lr += __shfl_xor(lr, 32, 64);
        const bool nonempty = l > 0.f;
        lse_v[nt] = nonempty ? (m_ref[nt] + fast_log2(l)) * LN2 : -INFINITY;
        float f = (nonempty && lr > 0.f) ? 1.0f / lr : 0.f;
        if (a.sink != nullptr && nonempty && head < a.H) f *= sigmoid(lse_v[nt] - a.sink[head]);
        // staging row hr holds O[head] with 16-byte chunk c at c ^ (hr % 16)
        const int hr = wave * NT * 16 + nt * 16 + n_e;
        __bf16* sp = hr < 64 ? s_tile0 + hr * C::DV : s_tile1 + (hr - 64) * C::DV;
#pragma unroll
        for (int mc = 0; mc < C::MC; ++mc) {
            const f32x4 v = oacc[mc][nt] * f;
            const int col = (mc * 16 + 4 * g_e) ^ ((hr & 15) << 3);
            st4(sp + col, cvt4(v[0], v[1], v[2], v[3]));
        }
        if (active && g_e == 0 && head < a.H) a.lse[(size_t)t * a.H + head] = lse_v[nt];
    }
    __syncthreads();
    // coalesced stores: HT rows of DV bf16, 16 bytes per thread per step
    const int nh = (a.H - h_wg) < C::HT ? (a.H - h_wg) : C::HT;
    constexpr int CPR = C::DV / 8;      // chunks per row
    for (int id = tid; id < nh * CPR; id += NTH) {
        const int r = id / CPR, ch = id - r * CPR;
        const __bf16* sp = r < 64 ? s_tile0 + r * C::DV : s_tile1 + (r - 64) * C::DV;
        *reinterpret_cast<u32x4*>(a.o + ((size_t)t * a.H + h_wg + r) * C::DV + ch * 8) =
            *reinterpret_cast<const u32x4*>(sp + ((ch * 8) ^ ((r & 15) << 3)));
    }
}

// Merge of the split partials, one wave per (token, head): with M the largest
// reference max among the splits that saw a valid slot and f_s = 2^(m_s - M),
//   O = sum_s f_s O_s / sum_s f_s lr_s,   LSE = (M + log2 sum_s f_s l_s) ln 2,
// the same normalisation (by the rounded weights) and LSE as one workgroup
// over all blocks; then the sink fold of the forward's epilogue.
// (nsplit <= 64: lane s holds split s's sums)
__global__ __launch_bounds__(256) void fwd_combine_kernel(FwdArgs a) {
    constexpr int DV = 512;
    const int row = (int)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= a.T * a.H) return;
    const int t = row / a.H, h = row - t * a.H;
    const size_t base = (size_t)t * a.nsplit * a.H + h;       // split s: base + s * H
    // lane s < nsplit holds split s's stats; M over the splits with a valid slot
    f32x4 st = zero4();
    if (lane < a.nsplit) st = *reinterpret_cast<const f32x4*>(a.spart + (base + (size_t)lane * a.H) * 4);
    float M = st[1] > 0.f ? st[0] : -INFINITY;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) M = fmaxf(M, __shfl_xor(M, m, 64));
    // lane s: its split's factor 2^(m_s - M) (0 without a valid slot)
    const float fs = (M != -INFINITY && st[1] > 0.f) ? exp2f(st[0] - M) : 0.f;
    f32x4 acc0 = zero4(), acc1 = zero4();
    float l = 0.f, lr = 0.f;
    if (M != -INFINITY) {
        // four splits' rows in flight, summed in split order
        for (int s0 = 0; s0 < a.nsplit; s0 += 4) {
            f32x4 x[4][2];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int s = s0 + k < a.nsplit ? s0 + k : a.nsplit - 1;
                const float* op = a.opart + (base + (size_t)s * a.H) * DV + 8 * lane;
                x[k][0] = *reinterpret_cast<const f32x4*>(op);
                x[k][1] = *reinterpret_cast<const f32x4*>(op + 4);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (s0 + k >= a.nsplit) break;
                const float f = __shfl(fs, s0 + k, 64);
                const float sl = __shfl(st[1], s0 + k, 64), slr = __shfl(st[2], s0 + k, 64);
                l += f * sl;
                lr += f * slr;
                acc0 += f * x[k][0];
                acc1 += f * x[k][1];
            }
        }
    }
    const bool nonempty = l > 0.f;
    const float lse = nonempty ? (M + log2f(l)) * LN2 : -INFINITY;
    float f = (nonempty && lr > 0.f) ? 1.0f / lr : 0.f;
    if (a.sink != nullptr && nonempty) f *= sigmoid(lse - a.sink[h]);
    const bf16x8 o = cvt8(acc0 * f, acc1 * f);
    *reinterpret_cast<u32x4*>(a.o + ((size_t)t * a.H + h) * DV + 8 * lane) = __builtin_bit_cast(u32x4, o);
    if (lane == 0) a.lse[(size_t)t * a.H + h] = lse;
}

template <int DQK, int NW, int NT>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    constexpr int HT = NW * NT * 16;
    if (a.nsplit > 1) {
        dim3 grid(a.T, (a.H + HT - 1) / HT, a.nsplit);
        hipLaunchKernelGGL((fwd_kernel<DQK, NW, NT, true>), grid, dim3(NW * 64), 0, stream, a);
        hipLaunchKernelGGL(fwd_combine_kernel, dim3((a.T * a.H + 3) / 4), dim3(256), 0, stream, a);
    } else {
        dim3 grid(a.T, (a.H + HT - 1) / HT);
        hipLaunchKernelGGL((fwd_kernel<DQK, NW, NT, false>), grid, dim3(NW * 64), 0, stream, a);
    }
    return hipGetLastError();
}

hipError_t launch_fwd(int d_qk, const FwdArgs& a, hipStream_t stream) {
    // head tile: 4 waves x 32 heads (H > 64) or 4 waves x 16 heads; with
    // split KV always 16 heads per wave (FWD_SPLIT_HEAD_TILE)
    static_assert(FWD_SPLIT_HEAD_TILE == 64, "the split forward runs 4 waves x 16 heads");
    const bool wide = a.H > 64 && a.nsplit <= 1;
    if (d_qk == 576)
        return wide ? launch_fwd_t<576, 4, 2>(a, stream) : launch_fwd_t<576, 4, 1>(a, stream);
    return wide ? launch_fwd_t<512, 4, 2>(a, stream) : launch_fwd_t<512, 4, 1>(a, stream);
}

}  // namespace smla
