// C ABI entry points: argument validation, workspace layout and kernel
// sequencing on the caller's stream.  No allocation; the only global state is
// the per-GPU scratch array of li_topk_sfa_noalloc and its device addresses.
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace lisfa {

hipError_t li_score_dispatch(const IndexerDev& a, int D_I, int dtype, int qg, float* scores, int64_t ld,
                             int64_t max_visible, hipStream_t stream);
hipError_t topk_dispatch(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K,
                         int32_t* idx, void* ws, hipStream_t stream);
hipError_t topk_candidates_dispatch(const float* scores, int64_t ld, const int32_t* row_pos, int R, int K,
                                    const int32_t* pos_offset, int32_t* cand_pos, float* cand_score, void* ws,
                                    hipStream_t stream);
hipError_t topk_merge_dispatch(const float* cand_score, const int32_t* cand_pos, int64_t ldc, int R, int n, int K,
                               int ordered, int32_t* idx, float* idx_score, hipStream_t stream);
int topk_slices(int64_t ld, int K);
size_t topk_workspace_bytes(int R, int64_t ld, int K);
hipError_t sfa_dispatch(const MlaDev& a, int D_latent, int kv_mode, __bf16* out, float* out_f32, float* lse, void* ws,
                        hipStream_t stream);
size_t sfa_workspace_bytes(int R, int K, int H, int D_latent);
size_t li_topk_workspace_bytes(int R);
int li_topk_fused_chunks(const IndexerDev& a, int D_I, int dtype, int qg, int64_t ld, int K, int layer);
hipError_t li_topk_dispatch(const IndexerDev& a, int D_I, int dtype, int qg, int64_t ld, int K, int32_t* idx,
                            void* ws, size_t ws_bytes, int layer, hipStream_t st);
hipError_t sfa_partial_dispatch(const MlaDev& a, const int32_t* range, int D_latent, int kv_mode, float* out_f32,
                                float* lse, void* ws, hipStream_t stream);
size_t sfa_partial_workspace_bytes(int R, int K, int H, int D_latent, int with_range);
hipError_t lse_combine_dispatch(const float* part_o, const float* part_lse, int G, int R, int H, int D, __bf16* out,
                                float* lse, hipStream_t stream);
hipError_t zigzag_restore_dispatch(const void* src, void* dst, int64_t n, int G, int64_t row_bytes,
                                   hipStream_t stream);
void zigzag_share_ranges(int64_t n, int G, int g, int64_t* r4);
hipError_t q_quant_dispatch(const void* q, int R, int n, int mx, void* out, void* scale_out, hipStream_t stream);
hipError_t prolog_dispatch(const void* q, int R, int n, int mx, void* q_out, void* q_scale_out, const void* k, int T,
                           int D_I, const float* gamma, const float* beta, float eps, int normalize,
                           const int32_t* tok_seq, const int32_t* tok_pos, const CacheDev& c, int dtype,
                           hipStream_t stream);
hipError_t k_store_dispatch(const void* k, int T, int D_I, const float* gamma, const float* beta, float eps,
                            int normalize, const int32_t* tok_seq, const int32_t* tok_pos, const CacheDev& c,
                            int dtype, hipStream_t stream);

namespace {

constexpr int64_t kScoreScratchCap = 256ll << 20;  // bytes of scores per fused chunk

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int check_cache(const lisfa_cache& c, int width) {
    if (!c.data) return LISFA_ERR_NULL_ARG;
    if (c.dtype != LISFA_BF16 && c.dtype != LISFA_FP8_E4M3 && c.dtype != LISFA_MXFP8 && c.dtype != LISFA_FP8_TILE128)
        return LISFA_ERR_BAD_DTYPE;
    const int elt = c.dtype == LISFA_BF16 ? 2 : 1;
    if (c.row_stride_bytes < width * elt || c.row_stride_bytes % 16 != 0) return LISFA_ERR_BAD_SHAPE;
    if (!aligned(c.data, 16)) return LISFA_ERR_BAD_SHAPE;
    if (c.num_slots <= 0 || c.num_seqs <= 0) return LISFA_ERR_BAD_SHAPE;
    if (c.dtype == LISFA_FP8_E4M3) {
        if (!c.scale) return LISFA_ERR_NULL_ARG;
        if (c.scale_group_tokens < 1) return LISFA_ERR_BAD_SHAPE;
    }
    if (c.dtype == LISFA_MXFP8) {
        if (!c.scale) return LISFA_ERR_NULL_ARG;
        if (width % 32 != 0) return LISFA_ERR_BAD_SHAPE;
        if (!aligned(c.scale, 4)) return LISFA_ERR_BAD_SHAPE;
    }
    if (c.dtype == LISFA_FP8_TILE128) {
        if (!c.scale) return LISFA_ERR_NULL_ARG;
        if (!aligned(c.scale, 4)) return LISFA_ERR_BAD_SHAPE;
    }
    if (c.block_table) {
        if (c.block_size < 1 || c.block_size > (1 << 20) || (c.block_size & (c.block_size - 1)))
            return LISFA_ERR_BAD_SHAPE;
        if (c.bt_stride < 1) return LISFA_ERR_BAD_SHAPE;
    } else if (!c.seq_base_slot) {
        return LISFA_ERR_NULL_ARG;
    }
    return LISFA_OK;
}

// attention kernels' view of the latent cache format
int kv_mode(const lisfa_cache& c) {
    return c.dtype == LISFA_FP8_TILE128 ? 2 : c.dtype == LISFA_FP8_E4M3 ? 1 : 0;
}

CacheDev to_dev(const lisfa_cache& c) {
    CacheDev d;
    d.data = (const uint8_t*)c.data;
    d.num_slots = c.num_slots;
    d.scale = (c.dtype == LISFA_FP8_E4M3 || c.dtype == LISFA_FP8_TILE128) ? (const float*)c.scale : nullptr;
    d.mx_scale = c.dtype == LISFA_MXFP8 ? (const uint8_t*)c.scale : nullptr;
    d.block_table = c.block_table;
    d.seq_base = c.seq_base_slot;
    d.row_stride = c.row_stride_bytes;
    d.scale_group = c.scale_group_tokens < 1 ? 1 : c.scale_group_tokens;
    d.bs_shift = 0;
    if (c.block_table)
        while ((1 << d.bs_shift) < c.block_size) ++d.bs_shift;
    d.bt_stride = c.bt_stride;
    d.num_seqs = c.num_seqs;
    d.paged = c.block_table != nullptr;
    return d;
}

int check_indexer(const lisfa_indexer_args* a) {
    if (!a) return LISFA_ERR_NULL_ARG;
    if (a->R < 0 || a->max_visible < 0) return LISFA_ERR_BAD_SHAPE;
    if (a->H_I < 1 || a->H_I > 64) return LISFA_ERR_UNSUPPORTED;
    if (a->D_I != 32 && a->D_I != 128) return LISFA_ERR_UNSUPPORTED;
    if (a->rows_per_group < 1) return LISFA_ERR_BAD_SHAPE;
    if (a->R == 0) return LISFA_OK;
    if (!a->q || !a->w || !a->row_seq || !a->row_pos) return LISFA_ERR_NULL_ARG;
    int e = check_cache(a->k_cache, a->D_I);
    if (e) return e;
    if (a->k_cache.dtype == LISFA_FP8_TILE128) return LISFA_ERR_BAD_DTYPE;   // a latent-cache format
    if (a->k_cache.dtype == LISFA_MXFP8) {
        if (a->D_I != 128) return LISFA_ERR_UNSUPPORTED;
        if (!a->q_scale) return LISFA_ERR_NULL_ARG;
        if (!aligned(a->q, 16)) return LISFA_ERR_BAD_SHAPE;
    } else if (a->k_cache.dtype == LISFA_FP8_E4M3) {
        if (!a->q_scale) return LISFA_ERR_NULL_ARG;
        if (!aligned(a->q, 8)) return LISFA_ERR_BAD_SHAPE;
    } else if (!aligned(a->q, 16)) {
        return LISFA_ERR_BAD_SHAPE;
    }
    return LISFA_OK;
}

IndexerDev to_dev(const lisfa_indexer_args* a) {
    IndexerDev d;
    d.q = (const uint8_t*)a->q;
    const bool mx = a->k_cache.dtype == LISFA_MXFP8;
    d.q_scale = mx ? nullptr : (const float*)a->q_scale;
    d.q_mx_scale = mx ? (const uint8_t*)a->q_scale : nullptr;
    d.w = a->w;
    d.row_seq = a->row_seq;
    d.row_pos = a->row_pos;
    d.k = to_dev(a->k_cache);
    d.q_scale_per_head = a->q_scale_per_head;
    d.R = a->R;
    d.H_I = a->H_I;
    return d;
}

int check_mla(const lisfa_mla_args* a) {
    if (!a) return LISFA_ERR_NULL_ARG;
    if (a->R < 0) return LISFA_ERR_BAD_SHAPE;
    if (a->H < 1 || a->H > 128) return LISFA_ERR_UNSUPPORTED;
    if (!((a->D_latent == 512 && a->D_rope == 64) || (a->D_latent == 64 && a->D_rope == 16)))
        return LISFA_ERR_UNSUPPORTED;
    // the online softmax raises its running maximum with scale * max(q.k), which
    // needs a positive, finite scale
    if (!(a->softmax_scale > 0.f) || !(a->softmax_scale < __builtin_inff())) return LISFA_ERR_BAD_SHAPE;
    if (a->R == 0) return LISFA_OK;
    if (!a->q || !a->row_seq) return LISFA_ERR_NULL_ARG;
    if (!aligned(a->q, 16)) return LISFA_ERR_BAD_SHAPE;
    if (a->kv_cache.dtype == LISFA_MXFP8) return LISFA_ERR_BAD_DTYPE;
    return check_cache(a->kv_cache, a->D_latent + a->D_rope);
}

MlaDev to_dev(const lisfa_mla_args* a, const int32_t* idx, int K) {
    MlaDev d;
    d.q = (const uint8_t*)a->q;
    d.row_seq = a->row_seq;
    d.idx = idx;
    d.kv = to_dev(a->kv_cache);
    d.R = a->R;
    d.H = a->H;
    d.K = K;
    d.scale_log2 = a->softmax_scale * kLog2e;
    // at most one query row per sequence: no cached row is gathered twice by
    // different query rows, so the gathers go non-temporal (2.8 -> 5.3 TB/s for
    // scattered rows from HBM); rows that share sequences (prefill) keep the
    // ordinary loads, whose cached lines the other rows reuse
    d.gather_nt = a->R <= a->kv_cache.num_seqs ? 1 : 0;
    return d;
}

int hip_status(hipError_t e) { return e == hipSuccess ? LISFA_OK : LISFA_ERR_HIP; }

int64_t scores_ld(int64_t max_visible) { return (max_visible + 63) / 64 * 64; }

// rows per chunk of the fused call: as many as keep the scores of a chunk
// within score_cap bytes
int64_t fused_chunk_rows(int32_t R, int64_t max_visible, int64_t score_cap) {
    const int64_t ld = scores_ld(max_visible) > 0 ? scores_ld(max_visible) : 64;
    int64_t rc = score_cap / (ld * 4);
    if (rc >= R) return R;
    // chunks start on multiples of 16 rows: the indexer forms its row groups
    // (1, 8 or 16 rows, each dividing the caller's rows_per_group) from the
    // chunk start, so every group it forms stays inside one of the caller's
    // aligned groups
    rc = rc / 16 * 16;
    return rc < 16 ? 16 : rc;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace of the index step (scores + Top-K): the score chunk, or the
// exchange area of the fused kernel, at offset 0, then Top-K scratch.
struct IndexLayout {
    size_t cand, total;
};

IndexLayout index_layout(int32_t R, int64_t max_visible, int32_t K, int64_t score_cap = kScoreScratchCap) {
    IndexLayout L;
    const int64_t rc = fused_chunk_rows(R, max_visible, score_cap);
    const size_t sc = align256((size_t)rc * scores_ld(max_visible) * sizeof(float));
    const size_t lt = align256(li_topk_workspace_bytes(R));
    L.cand = sc > lt ? sc : lt;
    L.total = L.cand + align256(topk_workspace_bytes((int)rc, scores_ld(max_visible), K));
    return L;
}

struct FusedLayout {
    size_t idx, sfa, total;
};

FusedLayout fused_layout(int32_t R, int64_t max_visible, int32_t K, int32_t H, int32_t D_latent,
                         int64_t score_cap = kScoreScratchCap) {
    FusedLayout L;
    L.idx = index_layout(R, max_visible, K, score_cap).total;
    L.sfa = L.idx + align256((size_t)R * K * sizeof(int32_t));
    L.total = L.sfa + align256(sfa_workspace_bytes(R, K, H, D_latent));
    return L;
}

// Indices of validated indexer rows: one fused score + Top-K launch where the
// shape and format allow it (scores stay on chip; layer != 0: only where that
// is the faster path), else scores in row chunks of at most score_cap bytes
// followed by topk_select.  The workspace at w is laid out by index_layout
// with the same cap.
int index_rows(const lisfa_indexer_args* iargs, int32_t K, int32_t* idx, uint8_t* w, int64_t score_cap, int layer,
               hipStream_t st) {
    const int32_t R = iargs->R;
    const IndexLayout L = index_layout(R, iargs->max_visible, K, score_cap);
    float* scores = (float*)w;
    const int64_t ld = scores_ld(iargs->max_visible) > 0 ? scores_ld(iargs->max_visible) : 64;
    const int qg = (iargs->rows_per_group % 16 == 0) ? 16 : (iargs->rows_per_group % 8 == 0) ? 8 : 1;
    IndexerDev d = to_dev(iargs);
    if (iargs->max_visible > 0) {
        const hipError_t he =
            li_topk_dispatch(d, iargs->D_I, iargs->k_cache.dtype, qg, ld, K, idx, w, L.cand, layer, st);
        if (he == hipSuccess) return LISFA_OK;
        if (he != hipErrorNotSupported) return LISFA_ERR_HIP;
    }
    const int64_t rc = fused_chunk_rows(R, iargs->max_visible, score_cap);
    const int elt = iargs->k_cache.dtype == LISFA_BF16 ? 2 : 1;
    const bool mx = iargs->k_cache.dtype == LISFA_MXFP8;
    for (int64_t c0 = 0; c0 < R; c0 += rc) {
        const int64_t c1 = c0 + rc < R ? c0 + rc : R;
        IndexerDev dc = d;
        dc.R = (int32_t)(c1 - c0);
        dc.q = d.q + c0 * (int64_t)iargs->H_I * iargs->D_I * elt;
        dc.w = d.w + c0 * iargs->H_I;
        if (d.q_scale) dc.q_scale = d.q_scale + c0 * (iargs->q_scale_per_head ? iargs->H_I : 1);
        if (mx) dc.q_mx_scale = d.q_mx_scale + c0 * (int64_t)iargs->H_I * (iargs->D_I / 32);
        dc.row_seq = d.row_seq + c0;
        dc.row_pos = d.row_pos + c0;
        if (iargs->max_visible > 0) {
            hipError_t he = li_score_dispatch(dc, iargs->D_I, iargs->k_cache.dtype, qg, scores, ld,
                                              iargs->max_visible, st);
            if (he != hipSuccess) return LISFA_ERR_HIP;
        }
        hipError_t he = topk_dispatch(scores, ld, dc.row_pos, dc.R, K, idx + c0 * K, w + L.cand, st);
        if (he != hipSuccess) return LISFA_ERR_HIP;
    }
    return LISFA_OK;
}

int check_fused(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs, int32_t K, const void* out) {
    int e = check_indexer(iargs);
    if (e) return e;
    e = check_mla(margs);
    if (e) return e;
    if (K < 1) return LISFA_ERR_BAD_SHAPE;
    if (iargs->R != margs->R) return LISFA_ERR_BAD_SHAPE;
    if (iargs->R == 0) return LISFA_OK;
    if (!out) return LISFA_ERR_NULL_ARG;
    if (!aligned(out, 8)) return LISFA_ERR_BAD_SHAPE;
    return LISFA_OK;
}

// The layer on validated arguments, the index step as index_rows with the
// given score cap, with the workspace at w (laid out by fused_layout with the
// same cap).
int fused_run(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs, int32_t K, int32_t* idx_out, void* out,
              float* lse, uint8_t* w, int64_t score_cap, hipStream_t st) {
    const FusedLayout L = fused_layout(iargs->R, iargs->max_visible, K, margs->H, margs->D_latent, score_cap);
    int32_t* idx = idx_out ? idx_out : (int32_t*)(w + L.idx);
    const int e = index_rows(iargs, K, idx, w, score_cap, 1, st);
    if (e) return e;
    const MlaDev md = to_dev(margs, idx, K);
    return hip_status(sfa_dispatch(md, margs->D_latent, kv_mode(margs->kv_cache), (__bf16*)out,
                                   nullptr, lse, w + L.sfa, st));
}

// Scratch of the allocation-free fused entry point: one array per GPU, held
// until the process ends.  In host code `scratch` only names the array; its
// device address (one per GPU) comes from hipGetSymbolAddress, taken once per
// device with that device current.
constexpr size_t kNoAllocScratchBytes = LISFA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

uint8_t* noalloc_scratch(hipStream_t stream) {
    int dev = -1;
    if (stream != nullptr) {
        if (hipStreamGetDevice(stream, &dev) != hipSuccess) return nullptr;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return nullptr;
    }
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    static std::mutex mu;
    static uint8_t* ptr[kMaxDevices] = {};
    std::lock_guard<std::mutex> lock(mu);
    if (ptr[dev] == nullptr) {
        int cur = -1;
        if (hipGetDevice(&cur) != hipSuccess) return nullptr;
        if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || p == nullptr) return nullptr;
        ptr[dev] = (uint8_t*)p;
    }
    return ptr[dev];
}

int check_q_quant(const void* q, int32_t R, int32_t H_I, int32_t D_I, int32_t dtype, const void* q_out,
                  const void* q_scale_out) {
    if (R < 0 || H_I < 1 || H_I > 64) return LISFA_ERR_BAD_SHAPE;
    if (D_I != 32 && D_I != 128) return LISFA_ERR_UNSUPPORTED;
    if (dtype != LISFA_FP8_E4M3 && dtype != LISFA_MXFP8) return LISFA_ERR_BAD_DTYPE;
    if (R == 0) return LISFA_OK;
    if (!q || !q_out || !q_scale_out) return LISFA_ERR_NULL_ARG;
    if (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(q_scale_out, 4)) return LISFA_ERR_BAD_SHAPE;
    return LISFA_OK;
}

int check_k_store(const void* k, int32_t T, int32_t D_I, float eps, const int32_t* tok_seq, const int32_t* tok_pos,
                  const lisfa_cache* k_cache) {
    if (T < 0) return LISFA_ERR_BAD_SHAPE;
    if (D_I != 32 && D_I != 128) return LISFA_ERR_UNSUPPORTED;
    if (!k_cache) return LISFA_ERR_NULL_ARG;
    int e = check_cache(*k_cache, D_I);
    if (e) return e;
    if (k_cache->dtype == LISFA_FP8_TILE128) return LISFA_ERR_BAD_DTYPE;   // a latent-cache format
    if (k_cache->dtype == LISFA_FP8_E4M3 && k_cache->scale_group_tokens != 1) return LISFA_ERR_BAD_SHAPE;
    if (!(eps >= 0.f)) return LISFA_ERR_BAD_SHAPE;
    if (T == 0) return LISFA_OK;
    if (!k || !tok_seq || !tok_pos) return LISFA_ERR_NULL_ARG;
    if (!aligned(k, 4) || (k_cache->dtype == LISFA_FP8_E4M3 && !aligned(k_cache->scale, 4))) return LISFA_ERR_BAD_SHAPE;
    return LISFA_OK;
}


}  // namespace
}  // namespace lisfa

using namespace lisfa;

extern "C" {

int32_t lisfa_abi_version(void) { return 1; }

size_t lisfa_struct_size(int32_t which) {
    switch (which) {
        case 0: return sizeof(lisfa_cache);
        case 1: return sizeof(lisfa_indexer_args);
        case 2: return sizeof(lisfa_mla_args);
        default: return 0;
    }
}

const char* lisfa_status_string(int32_t s) {
    switch (s) {
        case LISFA_OK: return "ok";
        case LISFA_ERR_NULL_ARG: return "a required pointer argument is NULL";
        case LISFA_ERR_BAD_SHAPE: return "a size, stride, alignment or layout argument is invalid";
        case LISFA_ERR_BAD_DTYPE: return "unsupported element type";
        case LISFA_ERR_WORKSPACE: return "workspace too small";
        case LISFA_ERR_HIP: return "HIP launch error";
        case LISFA_ERR_UNSUPPORTED: return "unsupported head count or head dimension";
        default: return "unknown status";
    }
}

size_t lisfa_workspace_size(int32_t op, int32_t R, int64_t max_visible, int32_t K, int32_t H,
                            int32_t D_latent) {
    if (R < 0 || K < 1) return 0;
    switch (op) {
        case LISFA_OP_TOPK:
        case LISFA_OP_TOPK_CANDIDATES: return topk_workspace_bytes(R, max_visible, K);
        case LISFA_OP_SPARSE_MLA: return sfa_workspace_bytes(R, K, H, D_latent);
        case LISFA_OP_FUSED: return fused_layout(R, max_visible, K, H, D_latent).total;
        case LISFA_OP_SPARSE_MLA_PARTIAL: return sfa_partial_workspace_bytes(R, K, H, D_latent, 1);
        case LISFA_OP_LI_TOPK: return index_layout(R, max_visible, K).total;
        default: return 0;
    }
}

int li_score(const lisfa_indexer_args* args, float* scores, int64_t ld_scores, lisfa_stream_t stream) {
    int e = check_indexer(args);
    if (e) return e;
    if (args->R == 0 || args->max_visible == 0) return LISFA_OK;
    if (!scores) return LISFA_ERR_NULL_ARG;
    if (ld_scores < args->max_visible) return LISFA_ERR_BAD_SHAPE;
    const IndexerDev d = to_dev(args);
    const int qg = (args->rows_per_group % 16 == 0) ? 16 : (args->rows_per_group % 8 == 0) ? 8 : 1;
    return hip_status(li_score_dispatch(d, args->D_I, args->k_cache.dtype, qg, scores, ld_scores,
                                        args->max_visible, (hipStream_t)stream));
}

int li_topk(const lisfa_indexer_args* args, int32_t K, int32_t* idx, void* ws, size_t ws_bytes,
            lisfa_stream_t stream) {
    int e = check_indexer(args);
    if (e) return e;
    if (K < 1) return LISFA_ERR_BAD_SHAPE;
    if (args->R == 0) return LISFA_OK;
    if (!idx) return LISFA_ERR_NULL_ARG;
    const IndexLayout L = index_layout(args->R, args->max_visible, K);
    if (L.total > 0 && (!ws || ws_bytes < L.total)) return LISFA_ERR_WORKSPACE;
    if (L.total > 0 && !aligned(ws, 256)) return LISFA_ERR_BAD_SHAPE;
    return index_rows(args, K, idx, (uint8_t*)ws, kScoreScratchCap, 0, (hipStream_t)stream);
}

int32_t li_topk_plan(const lisfa_indexer_args* args, int32_t K, int32_t layer) {
    const int e = check_indexer(args);
    if (e) return e;
    if (K < 1) return LISFA_ERR_BAD_SHAPE;
    if (args->R == 0 || args->max_visible == 0) return 0;
    const int qg = (args->rows_per_group % 16 == 0) ? 16 : (args->rows_per_group % 8 == 0) ? 8 : 1;
    return li_topk_fused_chunks(to_dev(args), args->D_I, args->k_cache.dtype, qg, scores_ld(args->max_visible), K,
                                layer != 0);
}

int topk_select(const float* scores, int64_t ld_scores, const int32_t* row_pos, int32_t R, int32_t K,
                int32_t* idx, void* ws, size_t ws_bytes, lisfa_stream_t stream) {
    if (R < 0 || K < 1 || ld_scores < 1) return LISFA_ERR_BAD_SHAPE;
    if (R == 0) return LISFA_OK;
    if (!scores || !row_pos || !idx) return LISFA_ERR_NULL_ARG;
    const size_t need = topk_workspace_bytes(R, ld_scores, K);
    void* w = nullptr;
    if (ws && need > 0) {
        if (ws_bytes < need) return LISFA_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return LISFA_ERR_BAD_SHAPE;
        w = ws;
    }
    return hip_status(topk_dispatch(scores, ld_scores, row_pos, R, K, idx, w, (hipStream_t)stream));
}

int topk_candidates(const float* scores, int64_t ld_scores, const int32_t* row_pos, int32_t R, int32_t K,
                    const int32_t* pos_offset, int32_t* cand_pos, float* cand_score, void* ws, size_t ws_bytes,
                    lisfa_stream_t stream) {
    if (R < 0 || K < 1 || ld_scores < 1) return LISFA_ERR_BAD_SHAPE;
    if (R == 0) return LISFA_OK;
    if (!scores || !row_pos || !cand_pos || !cand_score) return LISFA_ERR_NULL_ARG;
    if (ld_scores > 65536) {
        if (topk_slices(ld_scores, K) == 0) return LISFA_ERR_UNSUPPORTED;
        if (!ws || ws_bytes < topk_workspace_bytes(R, ld_scores, K)) return LISFA_ERR_WORKSPACE;
        if (!aligned(ws, 16)) return LISFA_ERR_BAD_SHAPE;
    }
    return hip_status(topk_candidates_dispatch(scores, ld_scores, row_pos, R, K, pos_offset, cand_pos, cand_score,
                                               ws, (hipStream_t)stream));
}

int topk_merge(const float* cand_score, const int32_t* cand_pos, int64_t ld_cand, int32_t R, int32_t n, int32_t K,
               int32_t ordered, int32_t* idx, float* idx_score, lisfa_stream_t stream) {
    if (R < 0 || K < 1 || n < 0 || ld_cand < n) return LISFA_ERR_BAD_SHAPE;
    if (n > 16384 || (!ordered && K > 4096)) return LISFA_ERR_UNSUPPORTED;
    if (R == 0) return LISFA_OK;
    if (!idx || (n > 0 && (!cand_score || !cand_pos))) return LISFA_ERR_NULL_ARG;
    return hip_status(topk_merge_dispatch(cand_score, cand_pos, ld_cand, R, n, K, ordered != 0, idx, idx_score,
                                          (hipStream_t)stream));
}

int sparse_mla_attn(const lisfa_mla_args* args, const int32_t* idx, int32_t K, void* out, float* lse,
                    void* ws, size_t ws_bytes, lisfa_stream_t stream) {
    int e = check_mla(args);
    if (e) return e;
    if (K < 1) return LISFA_ERR_BAD_SHAPE;
    if (args->R == 0) return LISFA_OK;
    if (!idx || !out) return LISFA_ERR_NULL_ARG;
    const size_t need = sfa_workspace_bytes(args->R, K, args->H, args->D_latent);
    if (need > 0 && (!ws || ws_bytes < need)) return LISFA_ERR_WORKSPACE;
    if (!aligned(out, 8)) return LISFA_ERR_BAD_SHAPE;
    const MlaDev d = to_dev(args, idx, K);
    return hip_status(sfa_dispatch(d, args->D_latent, kv_mode(args->kv_cache), (__bf16*)out,
                                   nullptr, lse, ws, (hipStream_t)stream));
}

int sparse_mla_attn_partial(const lisfa_mla_args* args, const int32_t* idx, int32_t K, const int32_t* range,
                            float* out, float* lse, void* ws, size_t ws_bytes, lisfa_stream_t stream) {
    int e = check_mla(args);
    if (e) return e;
    if (K < 1) return LISFA_ERR_BAD_SHAPE;
    if (args->R == 0) return LISFA_OK;
    if (!idx || !out || !lse) return LISFA_ERR_NULL_ARG;
    const size_t need = sfa_partial_workspace_bytes(args->R, K, args->H, args->D_latent, range != nullptr);
    if (need > 0 && (!ws || ws_bytes < need)) return LISFA_ERR_WORKSPACE;
    if (need > 0 && !aligned(ws, 256)) return LISFA_ERR_BAD_SHAPE;
    if (!aligned(out, 16)) return LISFA_ERR_BAD_SHAPE;
    const MlaDev d = to_dev(args, idx, K);
    return hip_status(sfa_partial_dispatch(d, range, args->D_latent, kv_mode(args->kv_cache), out,
                                           lse, ws, (hipStream_t)stream));
}

int lse_combine(const float* part_out, const float* part_lse, int32_t G, int32_t R, int32_t H, int32_t D_v,
                void* out, float* lse, lisfa_stream_t stream) {
    if (G < 1 || R < 0 || H < 1) return LISFA_ERR_BAD_SHAPE;
    if (D_v != 64 && D_v != 512) return LISFA_ERR_UNSUPPORTED;
    if ((int64_t)R * H > 0x7FFFFFFF) return LISFA_ERR_BAD_SHAPE;
    if (R == 0) return LISFA_OK;
    if (!part_out || !part_lse || !out) return LISFA_ERR_NULL_ARG;
    if (!aligned(part_out, 16) || !aligned(out, 16)) return LISFA_ERR_BAD_SHAPE;
    return hip_status(lse_combine_dispatch(part_out, part_lse, G, R, H, D_v, (__bf16*)out, lse, (hipStream_t)stream));
}

int lisfa_zigzag_share(int64_t n, int32_t G, int32_t g, int64_t* ranges) {
    if (!ranges) return LISFA_ERR_NULL_ARG;
    if (n < 0 || G < 1 || g < 0 || g >= G) return LISFA_ERR_BAD_SHAPE;
    if (n > ((int64_t)1 << 62) / (2 * (int64_t)G)) return LISFA_ERR_BAD_SHAPE;
    zigzag_share_ranges(n, G, g, ranges);
    return LISFA_OK;
}

int zigzag_restore(const void* src, void* dst, int64_t n, int32_t G, int64_t row_bytes, lisfa_stream_t stream) {
    if (n < 0 || G < 1 || row_bytes < 1) return LISFA_ERR_BAD_SHAPE;
    if (n > ((int64_t)1 << 40) / (2 * (int64_t)G)) return LISFA_ERR_BAD_SHAPE;
    if (n == 0) return LISFA_OK;
    if (!src || !dst) return LISFA_ERR_NULL_ARG;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst, len = (uintptr_t)(n * row_bytes);
    if (a < b + len && b < a + len) return LISFA_ERR_BAD_SHAPE;   // the buffers must not overlap
    return hip_status(zigzag_restore_dispatch(src, dst, n, G, row_bytes, (hipStream_t)stream));
}

int li_topk_sfa(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs, int32_t K, int32_t* idx_out,
                void* out, float* lse, void* ws, size_t ws_bytes, lisfa_stream_t stream) {
    int e = check_fused(iargs, margs, K, out);
    if (e || iargs->R == 0) return e;
    const FusedLayout L = fused_layout(iargs->R, iargs->max_visible, K, margs->H, margs->D_latent);
    if (!ws || ws_bytes < L.total) return LISFA_ERR_WORKSPACE;
    if (!aligned(ws, 256)) return LISFA_ERR_BAD_SHAPE;
    return fused_run(iargs, margs, K, idx_out, out, lse, (uint8_t*)ws, kScoreScratchCap, (hipStream_t)stream);
}

int li_topk_sfa_noalloc(const lisfa_indexer_args* iargs, const lisfa_mla_args* margs, int32_t K,
                        int32_t* idx_out, void* out, float* lse, lisfa_stream_t stream) {
    int e = check_fused(iargs, margs, K, out);
    if (e || iargs->R == 0) return e;
    // the largest score chunk whose layout fits the scratch array (more, smaller
    // chunks when it must); sizes whose smallest layout does not fit are refused
    int64_t cap = kScoreScratchCap;
    FusedLayout L = fused_layout(iargs->R, iargs->max_visible, K, margs->H, margs->D_latent, cap);
    while (L.total > kNoAllocScratchBytes && fused_chunk_rows(iargs->R, iargs->max_visible, cap) > 16) {
        cap /= 2;
        L = fused_layout(iargs->R, iargs->max_visible, K, margs->H, margs->D_latent, cap);
    }
    if (L.total > kNoAllocScratchBytes) return LISFA_ERR_WORKSPACE;
    uint8_t* w = noalloc_scratch((hipStream_t)stream);
    if (!w) return LISFA_ERR_HIP;
    return fused_run(iargs, margs, K, idx_out, out, lse, w, cap, (hipStream_t)stream);
}

int indexer_q_quant(const void* q, int32_t R, int32_t H_I, int32_t D_I, int32_t dtype, void* q_out,
                    void* q_scale_out, lisfa_stream_t stream) {
    const int e = check_q_quant(q, R, H_I, D_I, dtype, q_out, q_scale_out);
    if (e || R == 0) return e;
    return hip_status(q_quant_dispatch(q, R, H_I * D_I, dtype == LISFA_MXFP8, q_out, q_scale_out,
                                       (hipStream_t)stream));
}


int indexer_prolog(const void* q, int32_t R, int32_t H_I, int32_t D_I, int32_t q_dtype, void* q_out,
                   void* q_scale_out, const void* k, int32_t T, const float* gamma, const float* beta, float eps,
                   int32_t normalize, const int32_t* tok_seq, const int32_t* tok_pos, const lisfa_cache* k_cache,
                   lisfa_stream_t stream) {
    int e = check_q_quant(q, R, H_I, D_I, q_dtype, q_out, q_scale_out);
    if (e) return e;
    e = check_k_store(k, T, D_I, eps, tok_seq, tok_pos, k_cache);
    if (e) return e;
    if (R == 0 && T == 0) return LISFA_OK;
    return hip_status(prolog_dispatch(q, R, H_I * D_I, q_dtype == LISFA_MXFP8, q_out, q_scale_out, k, T, D_I, gamma,
                                      beta, eps, normalize != 0, tok_seq, tok_pos, to_dev(*k_cache), k_cache->dtype,
                                      (hipStream_t)stream));
}

int indexer_k_store(const void* k, int32_t T, int32_t D_I, const float* gamma, const float* beta, float eps,
                    int32_t normalize, const int32_t* tok_seq, const int32_t* tok_pos, const lisfa_cache* k_cache,
                    lisfa_stream_t stream) {
    int e = check_k_store(k, T, D_I, eps, tok_seq, tok_pos, k_cache);
    if (e) return e;
    if (T == 0) return LISFA_OK;
    return hip_status(k_store_dispatch(k, T, D_I, gamma, beta, eps, normalize != 0, tok_seq, tok_pos,
                                       to_dev(*k_cache), k_cache->dtype, (hipStream_t)stream));
}

}  // extern "C"
