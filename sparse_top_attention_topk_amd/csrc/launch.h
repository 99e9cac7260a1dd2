// Host-side launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace smla {

struct FwdArgs {
    const __bf16* q;
    const __bf16* kv;
    const int32_t* idx;
    const int32_t* len;
    const float* sink;
    __bf16* o;
    float* lse;
    int T, S_kv, H, W;
    float scale_log2;   // scale * log2(e)
    // split over each token's slot blocks (nsplit > 1): split s runs blocks
    // [s * bps, (s + 1) * bps) and writes partials, which a combine merges
    int nsplit, bps;
    float* opart;       // [T, nsplit, H, 512] fp32: unnormalised O of each split
    float* spart;       // [T, nsplit, H, 4] fp32: reference max (log2), sum, rounded sum, 0
};

struct BwdArgs {
    const __bf16* q;
    const __bf16* kv;
    const __bf16* dO;
    const float* lse;
    const float* delta;
    float* delta_out; // [T, H]: Delta written by the kernel that computes it (exact pass, or
                      // the S/dP kernel when o is set)
    const __bf16* o;  // [T, H, d_v] or NULL: the S/dP kernel computes Delta = sum O dO itself
    const int32_t* idx;
    const int32_t* len;
    const float* sink;
    __bf16* dq;
    float* dkv;
    // workspace, sized for one chunk of Tc tokens (tokens t0 .. t0 + Tc - 1;
    // "local" token index t - t0)
    __bf16* ws_p;     // [Tc, H, Wp] bf16: P
    __bf16* ws_ds;    // [Tc, H, Wp] bf16: scale * dS
    int* chunk_cnt;   // [nsub, S_kv]: per sub-chunk of the chunk, slots naming each row
    int* row_cnt;     // [S_kv]: valid slots of the chunk naming each KV row
    int* row_off;     // [S_kv + 1]: segment starts of the row-grouped list
    int* entries;     // [Tc * W]: local flat slot indices (t - t0) * Wp + j, grouped by row
    uint32_t* partial; // [Tc * Wp] rows of 2 * d_qk bytes: per-slot dKV contributions, 4-value blocks
    int* part_off;    // [S_kv + 1]: first reduce part of each row
    int* part_row;    // [max_parts]: row of each reduce part
    float* part_sum;  // [max_parts, d_qk] fp32: sums of the parts
    int max_parts;
    int T, S_kv, H, W, Wp;
    int t0, Tc;       // the chunk: its first token and its token count
    int nsub;         // sub-chunks of the chunk in the index inversion
    int tchunk;       // tokens per sub-chunk
    float scale, scale_log2;
    // split over each token's slot blocks (nsplit > 1, few tokens): split s
    // (blockIdx.z) of the S/dP, dQ and dKV kernels runs blocks
    // [s * bps, (s + 1) * bps); dQ then goes through fp32 partials
    int nsplit, bps;
    float* dq_part;   // [Tc, nsplit, H, d_qk] fp32 when nsplit > 1
};

// Rows of the KV set whose inversion counters one workgroup keeps in LDS
// (128 KB); larger sets are split into row ranges, one workgroup per range.
constexpr int INV_ROWS = 32768;

hipError_t launch_fwd(int d_qk, const FwdArgs& a, hipStream_t stream);
// head tile of the forward (heads per workgroup)
inline int fwd_head_tile(int H) { return H > 64 ? 128 : 64; }
// head tile of the forward with split KV (few tokens)
constexpr int FWD_SPLIT_HEAD_TILE = 64;
hipError_t launch_preprocess(const __bf16* o, const __bf16* dO, float* delta, int rows,
                             hipStream_t stream);
// Delta[t, h] = sum_j P_j dP_j (uses q, kv, dO, lse, idx, len, sink, delta_out)
hipError_t launch_delta_exact(int d_qk, const BwdArgs& a, hipStream_t stream);
// ev: NULL, or SMLA_BWD_STAGES + 1 events recorded at the stage boundaries
hipError_t launch_bwd(int d_qk, const BwdArgs& a, float* d_sink, hipStream_t stream,
                      hipEvent_t* ev);

}  // namespace smla
