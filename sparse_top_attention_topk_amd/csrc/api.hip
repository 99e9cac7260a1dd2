// C ABI of libsmla: argument validation and kernel dispatch.  Nothing here
// allocates, frees or synchronises; every kernel goes to the caller's stream.
#include "../../include/smla.h"
#include "common.h"
#include "launch.h"

#include <mutex>

// The fixed scratch of smla_bwd_noalloc: one array per GPU, held from the
// library's load until the process ends.  Host code never uses this name as
// an address (on the host it is a stand-in): the device address of each GPU's
// copy comes from hipGetSymbolAddress on that GPU and is kept in
// g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[SMLA_NOALLOC_SCRATCH_BYTES];

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

smla_status check_dims(const smla_dims* d) {
    if (d == nullptr) return SMLA_ERR_NULL;
    if (d->T < 0 || d->S_kv < 1 || d->H < 1 || d->W < 1) return SMLA_ERR_SHAPE;
    if ((d->d_qk != 512 && d->d_qk != 576) || d->d_v != 512 || d->H > 128)
        return SMLA_ERR_UNSUPPORTED;
    // KV rows are addressed with 32-bit byte offsets; slot positions of a
    // row with 32-bit offsets as well
    if ((int64_t)d->S_kv * d->d_qk * 2 > INT32_MAX || d->W > SMLA_MAX_W) return SMLA_ERR_UNSUPPORTED;
    if (!(d->scale == d->scale) || d->scale == INFINITY || d->scale == -INFINITY)
        return SMLA_ERR_SHAPE;
    return SMLA_OK;
}

size_t round_up_blk(int W) { return ((size_t)W + smla::BLK - 1) / smla::BLK * smla::BLK; }

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Sub-chunks of a token chunk of C tokens in the index inversion: at most
// 256, and at most 16M counters in all (nsub x S_kv), so the counters stay
// within 64 MB for any number of KV rows.
int inversion_subchunks(const smla_dims* d, int C) {
    int64_t n = 256;
    const int64_t cap = ((int64_t)1 << 24) / d->S_kv;
    if (n > cap) n = cap > 0 ? cap : 1;
    if (n > C) n = C;
    return (int)n;
}

// Workspace layout of smla_bwd for token chunks of C tokens (each region
// 256-byte aligned):
//   P, scale*dS      bf16 [C, H, Wp] each (Wp = W rounded up to 64)
//   chunk_cnt        int32 [nsub, S_kv]
//   row_cnt          int32 [S_kv]; row_off int32 [S_kv + 1]
//   entries          int32 [C * W]
//   partial          [C * Wp] rows of d_qk values in 4-value blocks (2 * d_qk bytes)
//   part_off         int32 [S_kv + 1]; part_row int32 [max_parts]
//   part_sum         fp32 [max_parts, d_qk], max_parts = C * W / 64 + min(S_kv, C * W)
//                    (a row named n times has ceil(n / 64) parts)
//   dq_part          fp32 [C, nsplit, H, d_qk] when the blocks are split (C < 128)
struct WsLayout {
    size_t p, ds, chunk, cnt, off, ent, part, poff, prow, psum, dqp, total;
    int max_parts, nsub, nsplit, bps;
};

// Splits of each token's slot blocks in the backward for chunks of C
// tokens: from 128 tokens on the chunk is run one workgroup per token; below,
// the blocks are split until one round of about 256 workgroups is filled
// (at most one split per block).
void bwd_split_for(const smla_dims* d, int C, int* nsplit, int* bps) {
    const int64_t nb = ((int64_t)d->W + smla::BLK - 1) / smla::BLK;
    int64_t s = C >= 128 ? 1 : 256 / C;
    if (s > nb) s = nb;
    if (s < 2) {
        *nsplit = 1;
        *bps = (int)nb;
        return;
    }
    const int64_t b = (nb + s - 1) / s;
    *bps = (int)b;
    *nsplit = (int)((nb + b - 1) / b);
}

WsLayout ws_layout(const smla_dims* d, int C) {
    WsLayout L;
    const size_t Wp = round_up_blk(d->W);
    const size_t pd = (size_t)C * d->H * Wp * sizeof(uint16_t);
    L.nsub = inversion_subchunks(d, C);
    const size_t cw = (size_t)C * d->W;
    L.p = 0;
    L.ds = align256(L.p + pd);
    L.chunk = align256(L.ds + pd);
    L.cnt = align256(L.chunk + (size_t)L.nsub * d->S_kv * sizeof(int32_t));
    L.off = align256(L.cnt + (size_t)d->S_kv * sizeof(int32_t));
    L.ent = align256(L.off + ((size_t)d->S_kv + 1) * sizeof(int32_t));
    L.part = align256(L.ent + cw * sizeof(int32_t));
    L.poff = align256(L.part + (size_t)C * Wp * d->d_qk * 2);
    const size_t mp = cw / 64 + ((size_t)d->S_kv < cw ? (size_t)d->S_kv : cw);
    L.max_parts = (int)mp;
    L.prow = align256(L.poff + ((size_t)d->S_kv + 1) * sizeof(int32_t));
    L.psum = align256(L.prow + mp * sizeof(int32_t));
    L.dqp = align256(L.psum + mp * d->d_qk * sizeof(float));
    bwd_split_for(d, C, &L.nsplit, &L.bps);
    const size_t dqp = L.nsplit > 1 ? (size_t)C * L.nsplit * d->H * d->d_qk * sizeof(float) : 0;
    L.total = align256(L.dqp + dqp);
    return L;
}

// ---- split forward: how many splits over each token's slot blocks.  A
// token takes one workgroup per head tile; with few tokens the GPU's 256
// CUs are not filled, so the split forward runs head tiles of 64 (more
// workgroups, each writing half the partial O of a 128-head tile) and splits
// the blocks until one round of about 256 workgroups (one per CU) is filled,
// at most one split per block: a second round costs more than the longer
// ranges, and every split adds its fp32 partial O to write and merge.
struct FwdSplit {
    int nsplit, bps, nb;
};

FwdSplit fwd_split_for(const smla_dims* d) {
    const int64_t nb = ((int64_t)d->W + smla::BLK - 1) / smla::BLK;
    const int ht = smla::fwd_head_tile(d->H);
    const int64_t wgs = (int64_t)d->T * ((d->H + ht - 1) / ht);
    if (wgs >= 128) return {1, (int)nb, (int)nb};
    // split: tiles of 64 heads (twice the workgroups at H > 64, each with
    // half the partial O to write)
    const int64_t wgs_split = (int64_t)d->T * ((d->H + smla::FWD_SPLIT_HEAD_TILE - 1) / smla::FWD_SPLIT_HEAD_TILE);
    int64_t s = 256 / wgs_split;
    if (s > nb) s = nb;
    if (s > 64) s = 64;                          // the merge keeps one split per lane
    if (s < 2) return {1, (int)nb, (int)nb};
    const int64_t bps = (nb + s - 1) / s;
    return {(int)((nb + bps - 1) / bps), (int)bps, (int)nb};
}

size_t fwd_split_bytes(const smla_dims* d, int nsplit) {
    if (nsplit <= 1) return 0;
    const size_t rows = (size_t)d->T * nsplit * d->H;
    return align256(rows * 512 * sizeof(float)) + align256(rows * 4 * sizeof(float));
}

// Largest chunk whose workspace fits in `bytes` (0 if not even one token's
// does).  Local slot indices (t - t0) * Wp + j and part counts stay in int32.
// The workspace grows with the chunk from 128 tokens on (no block split);
// below 128 it also holds the dQ shares of the split blocks, whose size is
// not monotone in the chunk, so the range below 256 is scanned.
int max_chunk(const smla_dims* d, size_t bytes) {
    const int64_t Wp = (int64_t)round_up_blk(d->W);
    int64_t hi = d->T;
    const int64_t lim = (INT32_MAX / 2) / Wp;
    if (hi > lim) hi = lim;
    if (hi < 1) return 0;
    if (ws_layout(d, (int)hi).total <= bytes) return (int)hi;
    if (hi > 256 && ws_layout(d, 256).total <= bytes) {
        int64_t lo = 256;                  // fits; hi does not
        while (hi - lo > 1) {
            const int64_t mid = (lo + hi) / 2;
            if (ws_layout(d, (int)mid).total <= bytes) lo = mid;
            else hi = mid;
        }
        return (int)lo;
    }
    for (int64_t c = hi < 255 ? hi : 255; c >= 1; --c)
        if (ws_layout(d, (int)c).total <= bytes) return (int)c;
    return 0;
}

// Tokens per chunk for a workspace of `bytes`: the largest chunk that fits,
// evened out over the same number of chunks when the even size fits too (it
// may not: below 128 tokens a smaller chunk can need more, for the dQ shares
// of its split blocks).  0 if not even one token's chunk fits.  The result
// always satisfies ws_layout(d, C).total <= bytes.
int chunk_tokens(const smla_dims* d, size_t bytes) {
    const int cmax = max_chunk(d, bytes);
    if (cmax == 0) return 0;
    const int64_t n = ((int64_t)d->T + cmax - 1) / cmax;
    const int even = (int)(((int64_t)d->T + n - 1) / n);
    return ws_layout(d, even).total <= bytes ? even : cmax;
}

constexpr int MAX_DEVICES = 64;
void* g_scratch_ptr[MAX_DEVICES] = {};
std::mutex g_scratch_mu;

// The current device's scratch address, looked up once per device with that
// device current (the first smla_bwd_noalloc call on it).
smla_status scratch_for_current_device(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SMLA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) {
            (void)hipGetLastError();
            return SMLA_ERR_LAUNCH;
        }
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return SMLA_OK;
}

}  // namespace

extern "C" {

const char* smla_status_string(smla_status s) {
    switch (s) {
        case SMLA_OK: return "ok";
        case SMLA_ERR_NULL: return "a required pointer is NULL";
        case SMLA_ERR_SHAPE: return "a size is negative or inconsistent";
        case SMLA_ERR_UNSUPPORTED:
            return "unsupported sizes: d_qk must be 512 or 576, d_v 512, H at most 128, "
                   "S_kv * d_qk * 2 below 2^31 and W at most 2^24";
        case SMLA_ERR_ALIGN: return "a base pointer is not 16-byte aligned";
        case SMLA_ERR_WORKSPACE: return "workspace missing or smaller than one token's chunk needs";
        case SMLA_ERR_LAUNCH: return "kernel launch failed";
        case SMLA_ERR_SCRATCH:
            return "smla_bwd_noalloc: one token's chunk of this problem needs more than the library's "
                   "fixed scratch (SMLA_NOALLOC_SCRATCH_BYTES); use smla_bwd with a workspace";
    }
    return "unknown status";
}

static smla_status fwd_impl(const smla_dims* d, const void* q, const void* kv, const int32_t* topk_idxs,
                            const int32_t* topk_length, const float* attn_sink, void* o, float* lse,
                            void* workspace, size_t workspace_bytes, void* stream) {
    smla_status st = check_dims(d);
    if (st != SMLA_OK) return st;
    if (d->T == 0) return SMLA_OK;
    if (!q || !kv || !topk_idxs || !o || !lse) return SMLA_ERR_NULL;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(o)) return SMLA_ERR_ALIGN;
    if (workspace != nullptr && !aligned16(workspace)) return SMLA_ERR_ALIGN;
    smla::FwdArgs a = {};
    // split over the slot blocks as far as the workspace allows
    FwdSplit sp = workspace != nullptr ? fwd_split_for(d) : FwdSplit{1, 0, 0};
    while (sp.nsplit > 1 && fwd_split_bytes(d, sp.nsplit) > workspace_bytes) {
        const int s = sp.nsplit - 1;             // fewer splits, as even as the blocks allow
        sp.bps = (sp.nb + s - 1) / s;
        sp.nsplit = (sp.nb + sp.bps - 1) / sp.bps;
    }
    a.nsplit = sp.nsplit > 1 ? sp.nsplit : 1;
    a.bps = sp.bps;
    if (a.nsplit > 1) {
        const size_t rows = (size_t)d->T * a.nsplit * d->H;
        a.opart = static_cast<float*>(workspace);
        a.spart = reinterpret_cast<float*>(static_cast<char*>(workspace) + align256(rows * 512 * sizeof(float)));
    }
    a.q = static_cast<const __bf16*>(q);
    a.kv = static_cast<const __bf16*>(kv);
    a.idx = topk_idxs;
    a.len = topk_length;
    a.sink = attn_sink;
    a.o = static_cast<__bf16*>(o);
    a.lse = lse;
    a.T = d->T; a.S_kv = d->S_kv; a.H = d->H; a.W = d->W;
    a.scale_log2 = d->scale * smla::LOG2E;
    hipError_t e = smla::launch_fwd(d->d_qk, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

smla_status smla_fwd(const smla_dims* d, const void* q, const void* kv, const int32_t* topk_idxs,
                     const int32_t* topk_length, const float* attn_sink, void* o, float* lse,
                     void* stream) {
    return fwd_impl(d, q, kv, topk_idxs, topk_length, attn_sink, o, lse, nullptr, 0, stream);
}

size_t smla_fwd_splitkv_workspace_size(const smla_dims* d) {
    if (check_dims(d) != SMLA_OK || d->T == 0) return 0;
    return fwd_split_bytes(d, fwd_split_for(d).nsplit);
}

smla_status smla_fwd_splitkv(const smla_dims* d, const void* q, const void* kv, const int32_t* topk_idxs,
                             const int32_t* topk_length, const float* attn_sink, void* o, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream) {
    if (workspace == nullptr) workspace_bytes = 0;
    return fwd_impl(d, q, kv, topk_idxs, topk_length, attn_sink, o, lse,
                    workspace_bytes > 0 ? workspace : nullptr, workspace_bytes, stream);
}

smla_status smla_bwd_preprocess(const smla_dims* d, const void* o, const void* dO, float* delta,
                                void* stream) {
    smla_status st = check_dims(d);
    if (st != SMLA_OK) return st;
    if (d->T == 0) return SMLA_OK;
    if (!o || !dO || !delta) return SMLA_ERR_NULL;
    if (!aligned16(o) || !aligned16(dO)) return SMLA_ERR_ALIGN;
    hipError_t e = smla::launch_preprocess(static_cast<const __bf16*>(o),
                                           static_cast<const __bf16*>(dO), delta, d->T * d->H,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

smla_status smla_bwd_delta_exact(const smla_dims* d, const void* q, const void* kv, const void* dO,
                                 const float* lse, const int32_t* topk_idxs,
                                 const int32_t* topk_length, const float* attn_sink, float* delta,
                                 void* stream) {
    smla_status st = check_dims(d);
    if (st != SMLA_OK) return st;
    if (d->T == 0) return SMLA_OK;
    if (!q || !kv || !dO || !lse || !topk_idxs || !delta) return SMLA_ERR_NULL;
    if (!aligned16(q) || !aligned16(kv) || !aligned16(dO)) return SMLA_ERR_ALIGN;
    smla::BwdArgs a = {};
    a.q = static_cast<const __bf16*>(q);
    a.kv = static_cast<const __bf16*>(kv);
    a.dO = static_cast<const __bf16*>(dO);
    a.lse = lse;
    a.delta_out = delta;
    a.idx = topk_idxs;
    a.len = topk_length;
    a.sink = attn_sink;
    a.T = d->T; a.S_kv = d->S_kv; a.H = d->H; a.W = d->W;
    a.Wp = (int)round_up_blk(d->W);
    a.t0 = 0;
    a.Tc = d->T;
    a.scale = d->scale;
    a.scale_log2 = d->scale * smla::LOG2E;
    hipError_t e = smla::launch_delta_exact(d->d_qk, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

size_t smla_bwd_workspace_size(const smla_dims* d) {
    if (check_dims(d) != SMLA_OK || d->T == 0) return 0;
    // one chunk (every token at once) when that fits the default budget,
    // else balanced chunks within it; never less than one token's workspace
    const int whole = max_chunk(d, ws_layout(d, d->T).total);
    if (whole == d->T && ws_layout(d, d->T).total <= SMLA_BWD_DEFAULT_WORKSPACE)
        return ws_layout(d, d->T).total;
    const int c = chunk_tokens(d, SMLA_BWD_DEFAULT_WORKSPACE);
    return ws_layout(d, c > 0 ? c : 1).total;
}

int smla_bwd_chunk_tokens(const smla_dims* d, size_t workspace_bytes) {
    if (check_dims(d) != SMLA_OK || d->T == 0) return 0;
    return chunk_tokens(d, workspace_bytes);
}

// o == NULL: delta is an input (from the preprocess or the exact pass).
// o != NULL: the S/dP kernel computes Delta = sum O dO and writes it to delta.
static smla_status bwd_impl(const smla_dims* d, const void* q, const void* kv, const void* dO,
                            const void* o, const float* lse, float* delta, const int32_t* topk_idxs,
                            const int32_t* topk_length, const float* attn_sink, void* dq, float* dkv,
                            float* d_sink, void* workspace, size_t workspace_bytes, void* stream,
                            void* const* events) {
    smla_status st = check_dims(d);
    if (st != SMLA_OK) return st;
    if (!dkv) return SMLA_ERR_NULL;
    if (attn_sink && !d_sink) return SMLA_ERR_NULL;
    if (d->T > 0) {
        if (!q || !kv || !dO || !lse || !delta || !topk_idxs || !dq) return SMLA_ERR_NULL;
        if (!aligned16(q) || !aligned16(kv) || !aligned16(dO) || !aligned16(dq) || !aligned16(dkv))
            return SMLA_ERR_ALIGN;
        if (o != nullptr && !aligned16(o)) return SMLA_ERR_ALIGN;
        if (workspace == nullptr) return SMLA_ERR_WORKSPACE;
        if (!aligned16(workspace)) return SMLA_ERR_ALIGN;
    }
    // tokens per chunk: as many as the workspace given holds (balanced)
    int C = 1;
    if (d->T > 0) {
        C = chunk_tokens(d, workspace_bytes);
        // every region the kernels address lies inside the workspace given
        if (C == 0 || ws_layout(d, C).total > workspace_bytes) return SMLA_ERR_WORKSPACE;
    }
    smla::BwdArgs a = {};
    a.q = static_cast<const __bf16*>(q);
    a.kv = static_cast<const __bf16*>(kv);
    a.dO = static_cast<const __bf16*>(dO);
    a.lse = lse;
    a.delta = delta;
    a.o = static_cast<const __bf16*>(o);
    a.delta_out = o != nullptr ? delta : nullptr;
    a.idx = topk_idxs;
    a.len = topk_length;
    a.sink = attn_sink;
    a.dq = static_cast<__bf16*>(dq);
    a.dkv = dkv;
    a.T = d->T; a.S_kv = d->S_kv; a.H = d->H; a.W = d->W;
    a.Wp = (int)round_up_blk(d->W);
    a.t0 = 0;
    a.Tc = C;
    const WsLayout WL = ws_layout(d, C);
    a.nsub = WL.nsub;
    a.tchunk = (C + WL.nsub - 1) / WL.nsub;
    char* ws = static_cast<char*>(workspace);
    a.ws_p = reinterpret_cast<__bf16*>(ws + WL.p);
    a.ws_ds = reinterpret_cast<__bf16*>(ws + WL.ds);
    a.chunk_cnt = reinterpret_cast<int*>(ws + WL.chunk);
    a.row_cnt = reinterpret_cast<int*>(ws + WL.cnt);
    a.row_off = reinterpret_cast<int*>(ws + WL.off);
    a.entries = reinterpret_cast<int*>(ws + WL.ent);
    a.partial = reinterpret_cast<uint32_t*>(ws + WL.part);
    a.part_off = reinterpret_cast<int*>(ws + WL.poff);
    a.part_row = reinterpret_cast<int*>(ws + WL.prow);
    a.part_sum = reinterpret_cast<float*>(ws + WL.psum);
    a.max_parts = WL.max_parts;
    a.nsplit = WL.nsplit;
    a.bps = WL.bps;
    a.dq_part = WL.nsplit > 1 ? reinterpret_cast<float*>(ws + WL.dqp) : nullptr;
    a.scale = d->scale;
    a.scale_log2 = d->scale * smla::LOG2E;
    hipError_t e = smla::launch_bwd(d->d_qk, a, d_sink, static_cast<hipStream_t>(stream),
                                    reinterpret_cast<hipEvent_t*>(const_cast<void**>(events)));
    return e == hipSuccess ? SMLA_OK : SMLA_ERR_LAUNCH;
}

smla_status smla_bwd(const smla_dims* d, const void* q, const void* kv, const void* dO,
                     const float* lse, const float* delta, const int32_t* topk_idxs,
                     const int32_t* topk_length, const float* attn_sink, void* dq, float* dkv,
                     float* d_sink, void* workspace, size_t workspace_bytes, void* stream) {
    return bwd_impl(d, q, kv, dO, nullptr, lse, const_cast<float*>(delta), topk_idxs, topk_length, attn_sink,
                    dq, dkv, d_sink, workspace, workspace_bytes, stream, nullptr);
}

smla_status smla_bwd_from_o(const smla_dims* d, const void* q, const void* kv, const void* dO,
                            const void* o, const float* lse, float* delta, const int32_t* topk_idxs,
                            const int32_t* topk_length, const float* attn_sink, void* dq, float* dkv,
                            float* d_sink, void* workspace, size_t workspace_bytes, void* stream) {
    if (d != nullptr && d->T > 0 && o == nullptr) return SMLA_ERR_NULL;
    return bwd_impl(d, q, kv, dO, o, lse, delta, topk_idxs, topk_length, attn_sink, dq, dkv, d_sink,
                    workspace, workspace_bytes, stream, nullptr);
}

smla_status smla_bwd_profiled(const smla_dims* d, const void* q, const void* kv, const void* dO,
                              const float* lse, const float* delta, const int32_t* topk_idxs,
                              const int32_t* topk_length, const float* attn_sink, void* dq,
                              float* dkv, float* d_sink, void* workspace, size_t workspace_bytes,
                              void* stream, void* const* stage_events, int n_events) {
    if (stage_events == nullptr) return SMLA_ERR_NULL;
    if (n_events < SMLA_BWD_STAGES + 1) return SMLA_ERR_SHAPE;
    for (int i = 0; i <= SMLA_BWD_STAGES; ++i)
        if (stage_events[i] == nullptr) return SMLA_ERR_NULL;
    return bwd_impl(d, q, kv, dO, nullptr, lse, const_cast<float*>(delta), topk_idxs, topk_length, attn_sink,
                    dq, dkv, d_sink, workspace, workspace_bytes, stream, stage_events);
}

smla_status smla_bwd_noalloc(const smla_dims* d, const void* q, const void* kv, const void* dO,
                             const float* lse, const float* delta, const int32_t* topk_idxs,
                             const int32_t* topk_length, const float* attn_sink, void* dq, float* dkv,
                             float* d_sink, void* stream) {
    smla_status st = check_dims(d);
    if (st != SMLA_OK) return st;
    // the fixed scratch must hold at least one token's chunk
    if (d->T > 0 && max_chunk(d, SMLA_NOALLOC_SCRATCH_BYTES) == 0) return SMLA_ERR_SCRATCH;
    void* ws = nullptr;
    st = scratch_for_current_device(&ws);
    if (st != SMLA_OK) return st;
    return bwd_impl(d, q, kv, dO, nullptr, lse, const_cast<float*>(delta), topk_idxs, topk_length, attn_sink,
                    dq, dkv, d_sink, ws, SMLA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
