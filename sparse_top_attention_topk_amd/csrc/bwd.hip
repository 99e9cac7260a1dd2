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
// Kernels, in launch order:
//   preprocess   Delta = rowsum(O * dO) in fp32 (separate entry point)
//   zero_fill    dkv = 0
//   bwd_main     one workgroup per (token, 64-head tile): gathers the KV tile,
//                recomputes S, P, dP, dS with bf16 MFMA, accumulates dQ in
//                registers, and stores P and scale*dS (bf16) to the workspace
//                for the dKV kernel
//   bwd_dkv      one workgroup per token: contracts over all heads,
//                dKV_blk = (scale*dS)^T Q + P^T dO, and adds it to dkv rows of
//                the valid slots with fp32 atomics
//   dsink        one workgroup per head: deterministic sum over tokens
// An empty row (no valid slot) is a uniform branch: dQ = 0 is written and the
// token's q, dO, lse and delta are not read.
#include "kv_tile.h"
#include "launch.h"

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
    const bf16x8 x = ld8(o + off), y = ld8(dO + off);
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

__global__ __launch_bounds__(256) void zero_fill_kernel(float* __restrict__ p, size_t n) {
    size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    const size_t stride = (size_t)gridDim.x * 256 * 4;
    for (; i + 4 <= n; i += stride) *reinterpret_cast<f32x4*>(p + i) = zero4();
    for (; i < n; ++i) p[i] = 0.f;   // tail (n not a multiple of 4)
}


// ---------------------------------------------------------------------------
// Main backward kernel: S, P, dP, dS, dQ for 64 heads of one token.
// Each of the 4 waves owns 16 heads; Q and dO stay in registers as the B
// operands of S^T = K Q^T and dP^T = V dO^T; dQ^T accumulates in registers.
// ---------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(256, 1) void bwd_main_kernel(BwdArgs a) {
    constexpr int DV = 512;
    constexpr int KS = DQK / 32, KV_ = DV / 32, MC = DQK / 16;
    using Tile = KvTile<DQK>;
    __shared__ __attribute__((aligned(16))) __bf16 s_tile[Tile::ELEMS];
    __shared__ int s_row[BLK];

    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int t = a.T - 1 - (int)blockIdx.x;
    const int head = (int)blockIdx.y * 64 + wave * 16 + n;
    const bool active = (int)blockIdx.y * 64 + wave * 16 < a.H;   // wave-uniform
    const bool hv = head < a.H;
    const int L = row_length(a.len, t, a.W);
    const int nblk = (L + BLK - 1) / BLK;

    bf16x8 qop[KS], dop[KV_];
    float lse_log2 = 0.f, dlt = 0.f;
    if (nblk > 0) {
        const int hh = hv ? head : 0;
        const __bf16* qp = a.q + ((size_t)t * a.H + hh) * DQK + 8 * g;
        const __bf16* dp = a.dO + ((size_t)t * a.H + hh) * DV + 8 * g;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qop[ks] = hv ? ld8(qp + 32 * ks) : zero8();
#pragma unroll
        for (int ks = 0; ks < KV_; ++ks) dop[ks] = hv ? ld8(dp + 32 * ks) : zero8();
        if (hv) {
            const float l = a.lse[(size_t)t * a.H + head];
            const float lt = a.sink ? glae(l, a.sink[head]) : l;
            lse_log2 = lt * LOG2E;    // +inf for a saturating sink: every P is 0
            dlt = a.delta[(size_t)t * a.H + head];
        }
    }

    f32x4 dqacc[MC];
#pragma unroll
    for (int mc = 0; mc < MC; ++mc) dqacc[mc] = zero4();

    for (int b = 0; b < nblk; ++b) {
        __syncthreads();
        Tile::load_rows(s_row, a.idx, t, a.W, L, a.S_kv, b);
        __syncthreads();
        Tile::gather(s_tile, s_row, a.kv);
        __syncthreads();
        if (!active) continue;

        f32x4 sacc[4], dpacc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) { sacc[mt] = zero4(); dpacc[mt] = zero4(); }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                sacc[mt] = mfma16(Tile::row_op(s_tile, mt * 16, ks * 32, lane), qop[ks], sacc[mt]);
#pragma unroll
        for (int ks = 0; ks < KV_; ++ks)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                dpacc[mt] = mfma16(Tile::row_op(s_tile, mt * 16, ks * 32, lane), dop[ks], dpacc[mt]);

        // P and scale*dS; invalid slots (and padded heads) give exactly 0
        f32x4 pv[4], dsv[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const bool ok = hv && s_row[mt * 16 + 4 * g + i] >= 0;
                const float p = ok ? fast_exp2(sacc[mt][i] * a.scale_log2 - lse_log2) : 0.f;
                pv[mt][i] = p;
                dsv[mt][i] = p * (dpacc[mt][i] - dlt) * a.scale;
            }
        }
        if (hv) {
            const size_t base = ((size_t)t * a.H + head) * a.Wp + b * BLK + 4 * g;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                st4(a.ws_p + base + mt * 16, cvt4(pv[mt][0], pv[mt][1], pv[mt][2], pv[mt][3]));
                st4(a.ws_ds + base + mt * 16, cvt4(dsv[mt][0], dsv[mt][1], dsv[mt][2], dsv[mt][3]));
            }
        }
        const bf16x8 dsop0 = cvt8(dsv[0], dsv[1]);
        const bf16x8 dsop1 = cvt8(dsv[2], dsv[3]);
        // dQ^T += K^T (scale dS)^T
#pragma unroll
        for (int mc = 0; mc < MC; ++mc) {
            dqacc[mc] = mfma16(Tile::slot_op(s_tile, 0, mc * 16, lane), dsop0, dqacc[mc]);
            dqacc[mc] = mfma16(Tile::slot_op(s_tile, 32, mc * 16, lane), dsop1, dqacc[mc]);
        }
    }

    if (!active || !hv) return;
    __bf16* dqp = a.dq + ((size_t)t * a.H + head) * DQK + 4 * g;
#pragma unroll
    for (int mc = 0; mc < MC; ++mc)
        st4(dqp + mc * 16, cvt4(dqacc[mc][0], dqacc[mc][1], dqacc[mc][2], dqacc[mc][3]));
}

// ---------------------------------------------------------------------------
// dKV kernel: per token and 64-slot block,
//   dKV_blk[slot][c] = sum_h (scale dS)[h][slot] q[h][c] + P[h][slot] dO[h][c]
// Contraction over heads (padded to 128).  Wave w owns columns
// [w * DQK/4, (w+1) * DQK/4); q and dO for those columns are held in registers
// with heads in-lane (loaded once per token through an LDS transpose).
// ---------------------------------------------------------------------------
template <int DQK>
__global__ __launch_bounds__(256, 1) void bwd_dkv_kernel(BwdArgs a) {
    constexpr int DV = 512;
    constexpr int CW = DQK / 4;          // columns per wave
    constexpr int NTC = CW / 16;         // 16-column tiles per wave
    constexpr int HK = 4;                // k-steps of 32 heads (H padded to 128)
    constexpr int QRS = DQK + 8;         // staging row stride (q rows)
    constexpr int PRS = BLK + 8;         // P / dS tile row stride
    __shared__ __attribute__((aligned(16))) __bf16 s_stage[32 * QRS];
    __shared__ __attribute__((aligned(16))) __bf16 s_ds[128 * PRS];
    __shared__ __attribute__((aligned(16))) __bf16 s_p[128 * PRS];
    __shared__ int s_row[BLK];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, n = lane & 15;
    const int t = a.T - 1 - (int)blockIdx.x;
    const int L = row_length(a.len, t, a.W);
    const int nblk = (L + BLK - 1) / BLK;
    if (nblk == 0) return;                 // uniform: an empty row adds nothing
    const int c_wave = wave * CW;

    // q and dO with heads in-lane: lane (g, n) of k-step hk, column tile nt holds
    // X[32hk + 8g + j][c_wave + 16nt + n], j = 0..7
    bf16x8 qB[HK][NTC], dB[HK][NTC];
#pragma unroll
    for (int hk = 0; hk < HK; ++hk) {
#pragma unroll
        for (int pass = 0; pass < 2; ++pass) {
            const int D = pass == 0 ? DQK : DV;
            const __bf16* src = pass == 0 ? a.q : a.dO;
            __syncthreads();
            // stage rows (heads) 32hk .. 32hk+31 of this token, zeros past H
            for (int id = tid; id < 32 * (D / 8); id += 256) {
                const int r = id / (D / 8), ch = id - r * (D / 8);
                const int h = 32 * hk + r;
                u32x4 v = {0u, 0u, 0u, 0u};
                if (h < a.H) v = *reinterpret_cast<const u32x4*>(src + ((size_t)t * a.H + h) * D + ch * 8);
                *reinterpret_cast<u32x4*>(s_stage + r * QRS + ch * 8) = v;
            }
            __syncthreads();
            const int w = lane & 15;
            const int row = 8 * g + (w >> 2);
#pragma unroll
            for (int nt = 0; nt < NTC; ++nt) {
                const int col = c_wave + 16 * nt + 4 * (w & 3);
                bf16x8 v = zero8();
                if (pass == 0 || c_wave + 16 * nt < DV) {
                    const bf16x4 lo = lds_tr4(s_stage + row * QRS + col);
                    const bf16x4 hi = lds_tr4(s_stage + (row + 4) * QRS + col);
                    v = cat44(lo, hi);
                }
                if (pass == 0) qB[hk][nt] = v; else dB[hk][nt] = v;
            }
        }
    }

    for (int b = 0; b < nblk; ++b) {
        __syncthreads();
        KvTile<DQK>::load_rows(s_row, a.idx, t, a.W, L, a.S_kv, b);
        // P and scale*dS tiles [head][slot] for this block, zeros past H
        for (int id = tid; id < 2 * 128 * (BLK / 8); id += 256) {
            const int which = id / (128 * (BLK / 8));
            const int rem = id - which * 128 * (BLK / 8);
            const int h = rem / (BLK / 8), ch = rem - h * (BLK / 8);
            u32x4 v = {0u, 0u, 0u, 0u};
            if (h < a.H) {
                const __bf16* src = which ? a.ws_p : a.ws_ds;
                v = *reinterpret_cast<const u32x4*>(src + ((size_t)t * a.H + h) * a.Wp + b * BLK + ch * 8);
            }
            *reinterpret_cast<u32x4*>((which ? s_p : s_ds) + h * PRS + ch * 8) = v;
        }
        __syncthreads();

        f32x4 acc[4][NTC];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < NTC; ++nt) acc[mt][nt] = zero4();
        const int w = lane & 15;
#pragma unroll
        for (int hk = 0; hk < HK; ++hk) {
            const int row = 32 * hk + 8 * g + (w >> 2);
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int col = mt * 16 + 4 * (w & 3);
                // A operand [slot][head]: lane (g, slot n) holds heads 32hk+8g+j
                const bf16x8 aop_ds = cat44(lds_tr4(s_ds + row * PRS + col),
                                            lds_tr4(s_ds + (row + 4) * PRS + col));
                const bf16x8 aop_p = cat44(lds_tr4(s_p + row * PRS + col),
                                           lds_tr4(s_p + (row + 4) * PRS + col));
#pragma unroll
                for (int nt = 0; nt < NTC; ++nt) {
                    acc[mt][nt] = mfma16(aop_ds, qB[hk][nt], acc[mt][nt]);
                    if (c_wave + 16 * nt < DV) acc[mt][nt] = mfma16(aop_p, dB[hk][nt], acc[mt][nt]);
                }
            }
        }
        // scatter-add to the KV rows of the valid slots
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = s_row[mt * 16 + 4 * g + i];
                if (r >= 0) {
                    float* dst = a.dkv + (size_t)r * DQK + c_wave + n;
#pragma unroll
                    for (int nt = 0; nt < NTC; ++nt) unsafeAtomicAdd(dst + 16 * nt, acc[mt][nt][i]);
                }
            }
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
    for (int t = threadIdx.x; t < T; t += 256) {
        const float l = lse[(size_t)t * H + h];
        if (l == -INFINITY) continue;
        float ps;
        if (sk == -INFINITY) ps = 0.f;
        else if (sk == INFINITY && l == INFINITY) ps = 0.5f;
        else ps = sigmoid(sk - l);
        acc += ps * delta[(size_t)t * H + h];
    }
    s_part[threadIdx.x] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) s_part[threadIdx.x] += s_part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) d_sink[h] = -s_part[0];
}

hipError_t launch_bwd(int d_qk, const BwdArgs& a, float* d_sink, hipStream_t stream) {
    const size_t n_dkv = (size_t)a.S_kv * d_qk;
    const size_t want = (n_dkv + 1023) / 1024;
    const int zb = (int)(want < 1 ? 1 : (want > 4096 ? 4096 : want));
    hipLaunchKernelGGL(zero_fill_kernel, dim3(zb), dim3(256), 0, stream, a.dkv, n_dkv);
    if (a.T > 0) {
        dim3 gmain(a.T, (a.H + 63) / 64);
        if (d_qk == 576) {
            hipLaunchKernelGGL(bwd_main_kernel<576>, gmain, dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_dkv_kernel<576>, dim3(a.T), dim3(256), 0, stream, a);
        } else {
            hipLaunchKernelGGL(bwd_main_kernel<512>, gmain, dim3(256), 0, stream, a);
            hipLaunchKernelGGL(bwd_dkv_kernel<512>, dim3(a.T), dim3(256), 0, stream, a);
        }
    }
    if (a.sink != nullptr)
        hipLaunchKernelGGL(dsink_kernel, dim3(a.H), dim3(256), 0, stream, a.lse, a.delta, a.sink,
                           d_sink, a.T, a.H);
    return hipGetLastError();
}

}  // namespace smla
