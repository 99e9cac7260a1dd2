// Sparse MLA forward for gfx950: one workgroup per (token, head tile).
//
// Method ([flash-attn #2882] Agent Notes; [cuDNN-FE #785] Summary 2-3): for
// each token, the H query heads share the token's gathered KV rows.  Per block
// of 64 top-k slots the workgroup
//   1. resolves slot -> KV row (invalid slots -> -1) and gathers the rows into
//      an LDS tile (zeros for invalid slots);
//   2. computes S^T = K Q^T with bf16 MFMA (slots x heads, fp32 accumulate);
//      each wave owns NT x 16 heads and holds their Q in registers, padded
//      heads (h >= H) are zero rows, so any H in 1..128 runs without padded
//      copies in memory;
//   3. masks invalid slots to -inf before any exponential, then runs an
//      online softmax in the log2 domain (running max and sum per head);
//   4. accumulates O^T += V^T P^T with V^T read transposed from the same tile.
// The epilogue folds the sink: O = acc / l * sigmoid(lse - sink), where the
// sigmoid is the sink-free share of the mass ([cuDNN-FE #785] Why 3), and
// writes the sink-free natural-log LSE.  Empty rows write O = 0, LSE = -inf.
#include "kv_tile.h"
#include "launch.h"

namespace smla {


template <int DQK, int NT>
__global__ __launch_bounds__(256, 1) void fwd_kernel(FwdArgs a) {
    constexpr int DV = 512;
    constexpr int KS = DQK / 32;      // k-steps of S^T
    constexpr int MC = DV / 16;       // 16-column tiles of O^T
    using Tile = KvTile<DQK>;
    __shared__ __attribute__((aligned(16))) __bf16 s_tile[Tile::ELEMS];
    __shared__ int s_row[BLK];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int t = a.T - 1 - (int)blockIdx.x;          // longest rows first
    const int h_wave = (int)blockIdx.y * (4 * NT * 16) + wave * NT * 16;
    const bool active = h_wave < a.H;                 // wave-uniform
    const int L = row_length(a.len, t, a.W);
    const int nblk = (L + BLK - 1) / BLK;

    // Q as the B operand of S^T = K Q^T: lane (g, n) holds q[t, head, 32ks+8g..+7]
    bf16x8 qop[NT][KS];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int head = h_wave + nt * 16 + n;
        const __bf16* qp = a.q + ((size_t)t * a.H + (head < a.H ? head : 0)) * DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            qop[nt][ks] = (head < a.H && nblk > 0) ? ld8(qp + 32 * ks) : zero8();
    }

    f32x4 oacc[MC][NT];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) oacc[mc][nt] = zero4();
    float m_run[NT], l_run[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) { m_run[nt] = -INFINITY; l_run[nt] = 0.f; }

    for (int b = 0; b < nblk; ++b) {
        __syncthreads();
        Tile::load_rows(s_row, a.idx, t, a.W, L, a.S_kv, b);
        __syncthreads();
        Tile::gather(s_tile, s_row, a.kv);
        __syncthreads();
        if (!active) continue;

        // S^T tiles: 4 row tiles of 16 slots x NT column tiles of 16 heads
        f32x4 sacc[4][NT];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = zero4();
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const bf16x8 kop = Tile::row_op(s_tile, mt * 16, ks * 32, lane);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) sacc[mt][nt] = mfma16(kop, qop[nt][ks], sacc[mt][nt]);
            }
        }

        // mask invalid slots before the exponential; log2-domain scores
        float blk_max[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) blk_max[nt] = -INFINITY;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = s_row[mt * 16 + 4 * g + i] >= 0;
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    const float s = ok ? sacc[mt][nt][i] * a.scale_log2 : -INFINITY;
                    sacc[mt][nt][i] = s;
                    blk_max[nt] = fmaxf(blk_max[nt], s);
                }
            }
        }
        bf16x8 pop[2][NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            float mb = xor_max(xor_max(blk_max[nt], 16), 32);
            const float m_new = fmaxf(m_run[nt], mb);
            const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
            const float alpha = fast_exp2(m_run[nt] - m_use);
            float psum = 0.f;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = fast_exp2(sacc[mt][nt][i] - m_use);
                    sacc[mt][nt][i] = p;
                    psum += p;
                }
            l_run[nt] = l_run[nt] * alpha + psum;
            m_run[nt] = m_new;
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) oacc[mc][nt] *= alpha;
            pop[0][nt] = cvt8(sacc[0][nt], sacc[1][nt]);
            pop[1][nt] = cvt8(sacc[2][nt], sacc[3][nt]);
        }

        // O^T += V^T P^T
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
#pragma unroll
            for (int kk = 0; kk < 2; ++kk) {
                const bf16x8 vop = Tile::slot_op(s_tile, kk * 32, mc * 16, lane);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) oacc[mc][nt] = mfma16(vop, pop[kk][nt], oacc[mc][nt]);
            }
        }
    }

    if (!active) return;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int head = h_wave + nt * 16 + n;
        float l = l_run[nt];
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const bool nonempty = l > 0.f;
        const float lse = nonempty ? (m_run[nt] + fast_log2(l)) * LN2 : -INFINITY;
        float f = nonempty ? 1.0f / l : 0.f;
        if (a.sink != nullptr && nonempty && head < a.H) f *= sigmoid(lse - a.sink[head]);
        if (head < a.H) {
            __bf16* op = a.o + ((size_t)t * a.H + head) * DV + 4 * g;
#pragma unroll
            for (int mc = 0; mc < MC; ++mc) {
                const f32x4 v = oacc[mc][nt] * f;
                st4(op + mc * 16, cvt4(v[0], v[1], v[2], v[3]));
            }
            if (g == 0) a.lse[(size_t)t * a.H + head] = lse;
        }
    }
}

template <int DQK, int NT>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t stream) {
    dim3 grid(a.T, (a.H + 4 * NT * 16 - 1) / (4 * NT * 16));
    hipLaunchKernelGGL((fwd_kernel<DQK, NT>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

hipError_t launch_fwd(int d_qk, const FwdArgs& a, hipStream_t stream) {
    const bool wide = a.H > 64;
    if (d_qk == 576) return wide ? launch_fwd_t<576, 2>(a, stream) : launch_fwd_t<576, 1>(a, stream);
    return wide ? launch_fwd_t<512, 2>(a, stream) : launch_fwd_t<512, 1>(a, stream);
}

}  // namespace smla
