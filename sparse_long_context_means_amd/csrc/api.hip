// api.hip -- the C ABI of include/mpattn.h: argument validation, workspace
// layout and the launch sequence of each entry point.  Everything is enqueued
// on the caller's stream; nothing here allocates or synchronises.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "../../include/mpattn.h"
#include "kernels.hpp"

using namespace mpa;

extern "C" int32_t mpattn_max_clusters(const mpattn_params* p);

namespace {

constexpr int kD = 128;
constexpr size_t kAlign = 256;
constexpr int kMaxFinePerBlockHier = 2048;
constexpr int kMaxCoarsePerBlock = 64;
constexpr int kMaxDecodeClusters = 32768;  // selection bitmask held in LDS
constexpr int kUnitPathMinUnits = 16;      // fewer units: the split launches
constexpr size_t kStatusBytes = 8;         // two uint32 counters at the start of a decode workspace

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool is_hier(const mpattn_params* p) { return p->coarse_tokens_per_centroid > 0; }

mpattn_status check_params(const mpattn_params* p) {
    if (!p) return MPATTN_ERR_INVALID_ARG;
    if (p->batch < 1 || p->n_q_heads < 1 || p->n_kv_heads < 1 || p->capacity_tokens < 1 ||
        p->tokens_per_centroid < 1 || p->cluster_block < 1 || p->build_iters < 1 || p->update_iters < 1 ||
        p->splits < 0 || p->coarse_tokens_per_centroid < 0 || p->head_dim < 1)
        return MPATTN_ERR_INVALID_ARG;
    if (p->n_q_heads % p->n_kv_heads != 0) return MPATTN_ERR_INVALID_ARG;
    if (p->dtype != MPATTN_F32 && p->dtype != MPATTN_BF16) return MPATTN_ERR_INVALID_ARG;
    if (p->head_dim != kD) return MPATTN_ERR_UNSUPPORTED;
    const int G = p->n_q_heads / p->n_kv_heads;
    if (G != 1 && G != 2 && G != 4 && G != 8) return MPATTN_ERR_UNSUPPORTED;
    if (p->cluster_block > kMaxBlock) return MPATTN_ERR_UNSUPPORTED;
    if (p->tokens_per_centroid > p->cluster_block) return MPATTN_ERR_INVALID_ARG;
    if ((int64_t)p->batch * p->n_kv_heads > 65535) return MPATTN_ERR_UNSUPPORTED;  // grid y
    if (p->centroid_format != MPATTN_CENTROIDS_STORED && p->centroid_format != MPATTN_CENTROIDS_FP8)
        return MPATTN_ERR_INVALID_ARG;
    if (p->centroid_format == MPATTN_CENTROIDS_FP8 && (p->dtype != MPATTN_BF16 || is_hier(p)))
        return MPATTN_ERR_UNSUPPORTED;
    if (is_hier(p)) {
        if (p->coarse_iters < 1 || p->coarse_candidate_tokens < 0) return MPATTN_ERR_INVALID_ARG;
        if (ceil_div(p->cluster_block, p->tokens_per_centroid) > kMaxFinePerBlockHier ||
            ceil_div(p->cluster_block, p->coarse_tokens_per_centroid) > kMaxCoarsePerBlock)
            return MPATTN_ERR_UNSUPPORTED;
    }
    return MPATTN_OK;
}

int default_splits(int units) {
    int s = 1024 / (units > 0 ? units : 1);
    if (s < 1) s = 1;
    if (s > 64) s = 64;
    return s;
}

int splits_of(const mpattn_params* p) {
    return p->splits > 0 ? p->splits : default_splits(p->batch * p->n_kv_heads);
}

// Attend splits of a decode: the requested count, raised to the number of
// 256-cluster chunks of the approximate term (each split streams one).
int decode_splits(const mpattn_params* p, int32_t chunks) {
    const int s = splits_of(p);
    return s > chunks ? s : chunks;
}

// Most chunks a decode on a state of these capacities can stream.
int32_t max_chunks(const mpattn_params* p, int32_t Cmax, int32_t Dmax) {
    if (!is_hier(p)) return score_chunks(Cmax);
    const int32_t fine = Cmax < p->coarse_candidate_tokens ? Cmax : p->coarse_candidate_tokens;
    return score_chunks(Dmax) + score_chunks(fine);
}

bool unit_path(const mpattn_params* p);
bool hier_unit_path(const mpattn_params* p);

// Decode workspace regions.
struct DecodeWs {
    uint32_t* status;     // [2] counters the one-launch decodes add to (first bytes of the workspace)
    // per-unit path with several replicas: exchange words (tag << 32 | value);
    // they rely on the workspace holding zeros before its first decode
    uint64_t* xch;        // [U][Rx][Cmax] keys
    uint64_t* xpart;      // [U][Rx][G][d + 2] partials
    uint64_t* xcount;     // [U] arrival counters (the merging replica sets them back to 0)
    uint32_t* xepoch;     // [U] tag of each unit's last decode
    int32_t Rx;           // most replicas a decode on this layout uses
    uint64_t* hch;        // hierarchy in one launch: [U][Rh][Dmax] coarse-key words
    uint64_t* hpart;      // [U][Rh][G][d + 2] partial words
    uint64_t* hcount;     // [U] arrival words
    uint32_t* hepoch;     // [U]
    int32_t Rh;
    int32_t Rxh;          // the same when each query head is its own unit
    float* s;             // [U][Cmax][G] scores by cluster id
    int4* rs;             // [U][Cmax] cut records by item
    uint32_t* selmask;    // [U][Cw] selected clusters
    int32_t* sel_ids;     // [U][Cmax]
    int32_t* sel_off;     // [U][Cmax]
    int32_t* sel_pre;     // [U][Cmax + 1]
    int32_t* counts;      // [U][4]
    float* part_ml;       // [U][G][S][2]: one partial per attend split
    float* part_acc;      // [U][G][S][d]
    // hierarchy: coarse level and the fine items inside the candidates
    float* cs;            // [U][Dmax][G]
    int4* crs;            // [U][Dmax]
    uint32_t* cmask;      // [U][Dw]
    int32_t* csel_ids;    // [U][Dmax]
    int32_t* csel_off;    // [U][Dmax]
    int32_t* csel_pre;    // [U][Dmax + 1]
    int32_t* ccounts;     // [U][4]
    int32_t* fids;        // [U][Cmax]
    int32_t Cw, Dw;       // mask words
    size_t bytes;
};

DecodeWs layout_decode(const mpattn_params* p, int32_t Cmax, int32_t Dmax, char* base) {
    const size_t U = (size_t)p->batch * p->n_kv_heads;
    const size_t G = (size_t)(p->n_q_heads / p->n_kv_heads);
    const size_t S = (size_t)decode_splits(p, max_chunks(p, Cmax, Dmax));
    DecodeWs w{};
    w.Cw = (Cmax + 31) / 32;
    w.Dw = (Dmax + 31) / 32;
    size_t off = 0;
    auto take = [&](size_t bytes) -> char* {
        char* ptr = base ? base + off : nullptr;
        off += align_up(bytes);
        return ptr;
    };
    w.status = (uint32_t*)take(kStatusBytes);
    if (unit_path(p)) {
        // sized for both unit layouts: one unit per KV head (G heads each),
        // or one per query head (per-head selection)
        w.Rx = unit_replicas(mpattn_max_clusters(p), (int)U);
        w.Rxh = unit_replicas(mpattn_max_clusters(p), (int)(U * G));
        const size_t r1 = w.Rx > 1 ? U * w.Rx : 0, rh = w.Rxh > 1 ? U * G * w.Rxh : 0;
        if (r1 + rh > 0) {
            const size_t words = r1 > rh ? r1 : rh;
            const size_t parts = r1 * G > rh ? r1 * G : rh;
            w.xch = (uint64_t*)take(words * Cmax * 8);
            w.xpart = (uint64_t*)take(parts * (kD + 2) * 8);
            w.xcount = (uint64_t*)take(U * G * 8);
            w.xepoch = (uint32_t*)take(U * G * 4);
        }
    }
    if (hier_unit_path(p)) {
        w.Rh = hier_replicas((int)U);
        w.hch = (uint64_t*)take(U * w.Rh * (size_t)Dmax * 8);
        w.hpart = (uint64_t*)take(U * w.Rh * G * (kD + 2) * 8);
        w.hcount = (uint64_t*)take(U * 8);
        w.hepoch = (uint32_t*)take(U * 4);
    }
    w.s = (float*)take(U * Cmax * G * 4);
    w.rs = (int4*)take(U * Cmax * 16);
    w.selmask = (uint32_t*)take(U * w.Cw * 4);
    w.sel_ids = (int32_t*)take(U * Cmax * 4);
    w.sel_off = (int32_t*)take(U * Cmax * 4);
    w.sel_pre = (int32_t*)take(U * (Cmax + 1) * 4);
    w.counts = (int32_t*)take(U * 4 * 4);
    w.part_ml = (float*)take(U * G * S * 2 * 4);
    w.part_acc = (float*)take(U * G * S * kD * 4);
    if (is_hier(p)) {
        w.cs = (float*)take(U * Dmax * G * 4);
        w.crs = (int4*)take(U * Dmax * 16);
        w.cmask = (uint32_t*)take(U * w.Dw * 4);
        w.csel_ids = (int32_t*)take(U * Dmax * 4);
        w.csel_off = (int32_t*)take(U * Dmax * 4);
        w.csel_pre = (int32_t*)take(U * (Dmax + 1) * 4);
        w.ccounts = (int32_t*)take(U * 4 * 4);
        w.fids = (int32_t*)take(U * Cmax * 4);
    }
    w.bytes = off;
    return w;
}

// Dense decode workspace: partials [U][G][S][2] and [U][G][S][d].
size_t dense_ws_bytes(const mpattn_params* p) {
    const size_t U = (size_t)p->batch * p->n_kv_heads, G = (size_t)(p->n_q_heads / p->n_kv_heads);
    const size_t S = (size_t)dense_splits((int)U);
    return align_up(U * G * S * 2 * 4) + align_up(U * G * S * kD * 4);
}

mpattn_status hip_status(hipError_t e) { return e == hipSuccess ? MPATTN_OK : MPATTN_ERR_HIP; }

#define MPA_TRY(expr)                                  \
    do {                                               \
        hipError_t e_ = (expr);                        \
        if (e_ != hipSuccess) return MPATTN_ERR_HIP;   \
    } while (0)

mpattn_status check_state(const mpattn_params* p, const mpattn_state* st) {
    if (!st || !st->key_centroids || !st->value_centroids || !st->key_centroids_f32 || !st->sizes || !st->offsets ||
        !st->token_ids || !st->assign)
        return MPATTN_ERR_INVALID_ARG;
    if ((st->sorted_keys == nullptr) != (st->sorted_values == nullptr)) return MPATTN_ERR_INVALID_ARG;
    if (st->capacity_clusters < 1) return MPATTN_ERR_INVALID_ARG;
    if (p->centroid_format == MPATTN_CENTROIDS_FP8 &&
        (!st->key_codes || !st->key_scales || !st->value_codes || !st->value_scales))
        return MPATTN_ERR_INVALID_ARG;
    if (st->n_clustered < 0 || st->n_clusters < 0 || st->n_coarse < 0 || st->n_blocks < 0)
        return MPATTN_ERR_INVALID_ARG;
    if (is_hier(p)) {
        if (!st->coarse_key_centroids || !st->coarse_value_centroids || !st->coarse_key_centroids_f32 ||
            !st->coarse_sizes || !st->coarse_offsets || !st->coarse_members || !st->parent ||
            st->capacity_coarse < 1)
            return MPATTN_ERR_INVALID_ARG;
    }
    return MPATTN_OK;
}

// Clusters the blocks of `br` for every unit: init, `iters` Lloyd rounds,
// value centroids, optional sorted copy, optional coarse level.
mpattn_status run_blocks(const mpattn_params* p, const void* k, const void* v, mpattn_state* st, BlockRange br,
                         int iters, int32_t n_new_clusters, int32_t d_base, hipStream_t s) {
    const UnitGeom g{p->batch * p->n_kv_heads, p->capacity_tokens, st->capacity_clusters};
    MPA_TRY(launch_kmeans_init(p->dtype, k, g, br, p->seed, st->key_centroids_f32, st->key_centroids, s));
    for (int it = 0; it < iters; ++it) {
        MPA_TRY(launch_kmeans_assign(p->dtype, k, g, br, st->key_centroids, st->assign, s));
        MPA_TRY(launch_kmeans_csr(st->assign, g, br, st->sizes, st->offsets, st->token_ids, s));
        MPA_TRY(launch_segmented_mean(p->dtype, k, g, br.c_base, n_new_clusters, st->sizes, st->offsets,
                                      st->token_ids, st->key_centroids_f32, st->key_centroids, false, s));
    }
    MPA_TRY(launch_segmented_mean(p->dtype, v, g, br.c_base, n_new_clusters, st->sizes, st->offsets, st->token_ids,
                                  nullptr, st->value_centroids, true, s));
    if (p->centroid_format == MPATTN_CENTROIDS_FP8)
        MPA_TRY(launch_encode_codes(g, br.c_base, n_new_clusters, st->key_centroids, st->value_centroids,
                                    st->key_codes, st->key_scales, st->value_codes, st->value_scales, s));
    if (st->sorted_keys)
        MPA_TRY(launch_sorted_copy(p->dtype, k, v, g, br.p_base, br.n_end - br.p_base, st->token_ids,
                                   st->sorted_keys, st->sorted_values, s));
    if (is_hier(p)) {
        CoarseRange cr{br, d_base, p->coarse_tokens_per_centroid,
                       (int32_t)ceil_div(p->cluster_block, p->coarse_tokens_per_centroid), st->capacity_coarse};
        MPA_TRY(launch_coarse_build(p->dtype, g, cr, p->seed, p->coarse_iters, st->key_centroids,
                                    st->value_centroids, st->sizes, st->coarse_key_centroids_f32,
                                    st->coarse_key_centroids, st->coarse_value_centroids, st->coarse_sizes,
                                    st->parent, st->coarse_offsets, st->coarse_members, s));
    }
    return MPATTN_OK;
}

const char* kFlatStages[] = {"score", "select", "attend", "merge"};
const char* kUnitStages[] = {"unit"};

// The whole flat decode step of a unit in one workgroup (unit.hip) when the
// batch has enough units to fill the GPU and the split count is automatic.
bool unit_path(const mpattn_params* p) {
    if (is_hier(p) || p->splits > 0 || p->dtype != MPATTN_BF16) return false;
    const int G = p->n_q_heads / p->n_kv_heads;
    return unit_path_fits(p->dtype, G, mpattn_max_clusters(p)) && p->batch * p->n_kv_heads >= kUnitPathMinUnits;
}
const char* kHierStages[] = {"coarse_score", "coarse_select", "fine_score", "fine_select", "attend", "merge"};
const char* kHierUnitStages[] = {"hier_unit"};

// The whole hierarchical decode step of a unit in one launch (hier.hip):
// bf16 storage, automatic splits, groups of up to 4 query heads, at most
// 2048 coarse clusters and a candidate budget of at most 4096 tokens.
bool hier_unit_path(const mpattn_params* p) {
    if (!is_hier(p) || p->splits > 0 || p->dtype != MPATTN_BF16) return false;
    const int G = p->n_q_heads / p->n_kv_heads;
    return hier_path_fits(p->dtype, G, mpattn_max_coarse(p), p->coarse_candidate_tokens);
}

// Every argument of a decode but the workspace.
mpattn_status check_decode(const mpattn_params* p, const void* q, const void* k, const void* v,
                           int32_t n_tokens_total, const mpattn_state* st, int32_t token_budget, int32_t mode,
                           const float* out, int32_t first_stage, int32_t last_stage) {
    mpattn_status rc = check_params(p);
    if (rc != MPATTN_OK) return rc;
    if (!q || !k || !v || !out) return MPATTN_ERR_INVALID_ARG;
    if ((rc = check_state(p, st)) != MPATTN_OK) return rc;
    if (st->n_clusters < 1 || st->n_clusters > st->capacity_clusters) return MPATTN_ERR_INVALID_ARG;
    if (n_tokens_total < st->n_clustered || n_tokens_total > p->capacity_tokens) return MPATTN_ERR_INVALID_ARG;
    if (token_budget < 0) return MPATTN_ERR_INVALID_ARG;
    if (mode != MPATTN_MODE_MULTIPOLE && mode != MPATTN_MODE_OMIT && mode != MPATTN_MODE_PER_HEAD)
        return MPATTN_ERR_INVALID_ARG;
    const bool hier = is_hier(p);
    if (hier && mode != MPATTN_MODE_MULTIPOLE) return MPATTN_ERR_UNSUPPORTED;
    if ((mode == MPATTN_MODE_PER_HEAD || p->centroid_format == MPATTN_CENTROIDS_FP8) && !unit_path(p))
        return MPATTN_ERR_UNSUPPORTED;
    if (st->capacity_clusters > kMaxDecodeClusters || st->capacity_coarse > kMaxDecodeClusters)
        return MPATTN_ERR_UNSUPPORTED;
    if (hier && (st->n_coarse < 1 || st->n_coarse > st->capacity_coarse)) return MPATTN_ERR_INVALID_ARG;
    const int32_t n_stages = mpattn_decode_stage_count(p);
    if (first_stage < 0 || last_stage >= n_stages || first_stage > last_stage) return MPATTN_ERR_INVALID_ARG;
    return MPATTN_OK;
}

// ---- the decode entry point that allocates nothing: its workspace is this
//      file-scope device array (each GPU the library runs on holds its own
//      copy until the process ends).  In host code the array's name is only
//      a stand-in: its device address comes from hipGetSymbolAddress, once per
//      device, and only that address reaches kernels.
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kScratchDevices = 64;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct ScratchSlot {
    void* ptr;        // device address of `scratch` on this device
    uint64_t layout;  // layout of the decode that used it last
    bool used;
};
std::mutex g_scratch_mu;
ScratchSlot g_scratch[kScratchDevices];

__global__ void zero_fill_kernel(uint4* p, size_t n16) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
        p[i] = make_uint4(0u, 0u, 0u, 0u);
}

// FNV-1a over the fields that fix the decode workspace layout.
uint64_t layout_key(const mpattn_params* p, const mpattn_state* st) {
    const int64_t f[] = {p->batch, p->n_q_heads, p->n_kv_heads, p->dtype, p->capacity_tokens, p->tokens_per_centroid,
                         p->cluster_block, p->coarse_tokens_per_centroid, p->coarse_candidate_tokens, p->splits,
                         p->centroid_format, st->capacity_clusters, st->capacity_coarse};
    uint64_t h = 1469598103934665603ull;
    for (int64_t x : f) {
        for (int b = 0; b < 8; ++b) {
            h ^= (uint64_t)((x >> (8 * b)) & 0xff);
            h *= 1099511628211ull;
        }
    }
    return h;
}

// The device address of this device's scratch array, cleared (with a fill
// kernel on the caller's stream) on its first use and whenever the decode
// layout differs from the last call's: the array then holds no tag of
// another layout.
mpattn_status scratch_for(const mpattn_params* p, const mpattn_state* st, void** out, hipStream_t s) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return MPATTN_ERR_HIP;
    if (dev < 0 || dev >= kScratchDevices) return MPATTN_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ScratchSlot& slot = g_scratch[dev];
    if (!slot.ptr) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return MPATTN_ERR_HIP;
        slot.ptr = ptr;
    }
    const uint64_t key = layout_key(p, st);
    if (!slot.used || slot.layout != key) {
        hipLaunchKernelGGL(zero_fill_kernel, dim3(1024), dim3(256), 0, s, (uint4*)slot.ptr, kScratchBytes / 16);
        if (hipGetLastError() != hipSuccess) return MPATTN_ERR_HIP;
        slot.layout = key;
        slot.used = true;
    }
    *out = slot.ptr;
    return MPATTN_OK;
}

}  // namespace

extern "C" {

const char* mpattn_status_string(int32_t status) {
    switch (status) {
        case MPATTN_OK: return "ok";
        case MPATTN_ERR_INVALID_ARG: return "invalid argument";
        case MPATTN_ERR_UNSUPPORTED: return "unsupported configuration";
        case MPATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case MPATTN_ERR_CAPACITY: return "state capacity exceeded";
        case MPATTN_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

int32_t mpattn_max_clusters(const mpattn_params* p) {
    if (check_params(p) != MPATTN_OK) return 0;
    const int64_t N = p->capacity_tokens;
    const int64_t c = ceil_div(N, p->tokens_per_centroid) + ceil_div(N, p->cluster_block) + 1;
    return c > INT32_MAX ? 0 : (int32_t)c;
}

int32_t mpattn_max_coarse(const mpattn_params* p) {
    if (check_params(p) != MPATTN_OK || !is_hier(p)) return 0;
    const int64_t N = p->capacity_tokens;
    const int64_t c = ceil_div(N, p->coarse_tokens_per_centroid) + ceil_div(N, p->cluster_block) + 1;
    return c > INT32_MAX ? 0 : (int32_t)c;
}

size_t mpattn_workspace_bytes(const mpattn_params* p, int32_t capacity_clusters, int32_t capacity_coarse,
                              int32_t op) {
    if (check_params(p) != MPATTN_OK || capacity_clusters < 1 || capacity_coarse < 0) return (size_t)-1;
    if (op == MPATTN_OP_BUILD || op == MPATTN_OP_UPDATE) return 0;
    if (op == MPATTN_OP_DENSE) return dense_ws_bytes(p);
    if (op != MPATTN_OP_DECODE) return (size_t)-1;
    return layout_decode(p, capacity_clusters, capacity_coarse, nullptr).bytes;
}

mpattn_status mpattn_build_clusters(const mpattn_params* p, const void* k, const void* v, int32_t n_tokens,
                                    mpattn_state* st, void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    mpattn_status rc = check_params(p);
    if (rc != MPATTN_OK) return rc;
    if (!k || !v) return MPATTN_ERR_INVALID_ARG;
    if ((rc = check_state(p, st)) != MPATTN_OK) return rc;
    if (n_tokens < 1) return MPATTN_ERR_INVALID_ARG;
    if (n_tokens > p->capacity_tokens) return MPATTN_ERR_CAPACITY;
    const int32_t Bc = p->cluster_block, r = p->tokens_per_centroid;
    const int32_t nb = (int32_t)ceil_div(n_tokens, Bc);
    const int32_t cfull = (int32_t)ceil_div(Bc, r);
    const int32_t last = n_tokens - (nb - 1) * Bc;
    const int64_t C = (int64_t)(nb - 1) * cfull + ceil_div(last, r);
    if (C > st->capacity_clusters) return MPATTN_ERR_CAPACITY;
    int64_t D = 0;
    if (is_hier(p)) {
        const int32_t dfull = (int32_t)ceil_div(Bc, p->coarse_tokens_per_centroid);
        D = (int64_t)(nb - 1) * dfull + ceil_div(last, p->coarse_tokens_per_centroid);
        if (D > st->capacity_coarse) return MPATTN_ERR_CAPACITY;
    }
    const BlockRange br{0, n_tokens, 0, Bc, r, cfull, 0, nb};
    rc = run_blocks(p, k, v, st, br, p->build_iters, (int32_t)C, 0, (hipStream_t)stream);
    if (rc != MPATTN_OK) return rc;
    st->n_clustered = n_tokens;
    st->n_clusters = (int32_t)C;
    st->n_coarse = (int32_t)D;
    st->n_blocks = nb;
    return MPATTN_OK;
}

mpattn_status mpattn_update_window(const mpattn_params* p, const void* k, const void* v, int32_t n_tokens_total,
                                   mpattn_state* st, void* workspace, size_t workspace_bytes, void* stream) {
    (void)workspace;
    (void)workspace_bytes;
    mpattn_status rc = check_params(p);
    if (rc != MPATTN_OK) return rc;
    if (!k || !v) return MPATTN_ERR_INVALID_ARG;
    if ((rc = check_state(p, st)) != MPATTN_OK) return rc;
    if (n_tokens_total < st->n_clustered) return MPATTN_ERR_INVALID_ARG;
    if (n_tokens_total > p->capacity_tokens) return MPATTN_ERR_CAPACITY;
    const int32_t Bc = p->cluster_block, r = p->tokens_per_centroid;
    const int32_t nb = (n_tokens_total - st->n_clustered) / Bc;
    if (nb == 0) return MPATTN_OK;
    const int32_t cfull = (int32_t)ceil_div(Bc, r);
    const int64_t C = (int64_t)st->n_clusters + (int64_t)nb * cfull;
    if (C > st->capacity_clusters) return MPATTN_ERR_CAPACITY;
    int64_t D = st->n_coarse;
    if (is_hier(p)) {
        D += (int64_t)nb * ceil_div(Bc, p->coarse_tokens_per_centroid);
        if (D > st->capacity_coarse) return MPATTN_ERR_CAPACITY;
    }
    const BlockRange br{st->n_clustered, st->n_clustered + nb * Bc, st->n_clusters, Bc, r, cfull, st->n_blocks, nb};
    rc = run_blocks(p, k, v, st, br, p->update_iters, nb * cfull, st->n_coarse, (hipStream_t)stream);
    if (rc != MPATTN_OK) return rc;
    st->n_clustered += nb * Bc;
    st->n_clusters = (int32_t)C;
    st->n_coarse = (int32_t)D;
    st->n_blocks += nb;
    return MPATTN_OK;
}

int32_t mpattn_decode_stage_count(const mpattn_params* p) {
    if (check_params(p) != MPATTN_OK) return 0;
    return is_hier(p) ? (hier_unit_path(p) ? 1 : 6) : unit_path(p) ? 1 : 4;
}

const char* mpattn_decode_stage_name(const mpattn_params* p, int32_t stage) {
    const int32_t n = mpattn_decode_stage_count(p);
    if (stage < 0 || stage >= n) return nullptr;
    if (is_hier(p)) return hier_unit_path(p) ? kHierUnitStages[stage] : kHierStages[stage];
    return unit_path(p) ? kUnitStages[stage] : kFlatStages[stage];
}

mpattn_status mpattn_decode_ex(const mpattn_params* p, const void* q, const void* k, const void* v,
                               int32_t n_tokens_total, const mpattn_state* st, int32_t token_budget, int32_t mode,
                               float* out, void* workspace, size_t workspace_bytes, void* stream,
                               const mpattn_decode_debug* debug, int32_t first_stage, int32_t last_stage) {
    mpattn_status rc = check_decode(p, q, k, v, n_tokens_total, st, token_budget, mode, out, first_stage, last_stage);
    if (rc != MPATTN_OK) return rc;
    const bool hier = is_hier(p);
    const DecodeWs need = layout_decode(p, st->capacity_clusters, st->capacity_coarse, nullptr);
    if (!workspace || workspace_bytes < need.bytes) return MPATTN_ERR_WORKSPACE;
    const DecodeWs w = layout_decode(p, st->capacity_clusters, st->capacity_coarse, (char*)workspace);

    const hipStream_t s = (hipStream_t)stream;
    const int U = p->batch * p->n_kv_heads;
    const int G = p->n_q_heads / p->n_kv_heads;
    const int32_t bound0 = st->n_clusters < p->coarse_candidate_tokens ? st->n_clusters : p->coarse_candidate_tokens;
    const int32_t chunks = mode != MPATTN_MODE_MULTIPOLE
                               ? 0
                               : (hier ? score_chunks(st->n_coarse) + score_chunks(bound0) : score_chunks(st->n_clusters));
    const int S = decode_splits(p, chunks);
    const int32_t Cmax = st->capacity_clusters, Dmax = st->capacity_coarse, N = p->capacity_tokens;
    const int32_t C = st->n_clusters;
    const bool sorted = st->sorted_keys != nullptr;
    const int32_t want_pseudo = mode != MPATTN_MODE_OMIT ? 1 : 0;
    const int32_t bound = C < p->coarse_candidate_tokens ? C : p->coarse_candidate_tokens;
    const int32_t P = S;  // partial slots: one per attend split

    if (hier_unit_path(p)) {  // one stage
        const int R = hier_replicas(U);
        if (R != w.Rh) return MPATTN_ERR_WORKSPACE;
        HierArgs a{};
        a.q = q;
        a.kbar = st->key_centroids;
        a.vbar = st->value_centroids;
        a.sizes = st->sizes;
        a.offsets = st->offsets;
        a.Kx = sorted ? st->sorted_keys : k;
        a.Vx = sorted ? st->sorted_values : v;
        a.token_ids = sorted ? nullptr : st->token_ids;
        a.K = k;
        a.V = v;
        a.ckbar = st->coarse_key_centroids;
        a.cvbar = st->coarse_value_centroids;
        a.csizes = st->coarse_sizes;
        a.coffsets = st->coarse_offsets;
        a.cmembers = st->coarse_members;
        a.Cmax = Cmax;
        a.Dmax = Dmax;
        a.C = C;
        a.D = st->n_coarse;
        a.Nmax = N;
        a.n_clustered = st->n_clustered;
        a.n_total = n_tokens_total;
        a.budget = token_budget;
        a.cand_budget = p->coarse_candidate_tokens;
        a.pseudo = want_pseudo;
        a.Hq = p->n_q_heads;
        a.Hkv = p->n_kv_heads;
        a.out = out;
        a.xch = w.hch;
        a.xpart = w.hpart;
        a.xcount = w.hcount;
        a.xepoch = w.hepoch;
        a.status = w.status;
        a.dbg_selected = debug ? debug->selected : nullptr;
        a.dbg_candidates = debug ? debug->candidates : nullptr;
        a.dbg_exact = debug ? debug->exact_tokens : nullptr;
        a.rescore = debug ? debug->rescore : 0;
        MPA_TRY(launch_hier_decode(p->dtype, G, a, U, R, s));
        return MPATTN_OK;
    }
    if (unit_path(p)) {  // one stage
        // per-head selection: each query head is a unit of one head that
        // reads the clusters and cache of its KV head
        const bool per_head = mode == MPATTN_MODE_PER_HEAD;
        const int Uv = per_head ? U * G : U, Gv = per_head ? 1 : G;
        const int R = unit_replicas(C, Uv);
        if (R > 1 && R > (per_head ? w.Rxh : w.Rx)) return MPATTN_ERR_WORKSPACE;
        UnitArgs a{};
        a.q = q;
        a.kbar = st->key_centroids;
        a.vbar = st->value_centroids;
        a.sizes = st->sizes;
        a.offsets = st->offsets;
        a.Kx = sorted ? st->sorted_keys : k;
        a.Vx = sorted ? st->sorted_values : v;
        a.token_ids = sorted ? nullptr : st->token_ids;
        a.K = k;
        a.V = v;
        a.Cmax = Cmax;
        a.C = C;
        a.Nmax = N;
        a.n_clustered = st->n_clustered;
        a.n_total = n_tokens_total;
        a.budget = token_budget;
        a.pseudo = want_pseudo;
        a.Hq = p->n_q_heads;
        a.Hkv = per_head ? p->n_q_heads : p->n_kv_heads;
        a.ugroup = per_head ? G : 1;
        if (p->centroid_format == MPATTN_CENTROIDS_FP8) {
            a.kcodes = st->key_codes;
            a.kscales = st->key_scales;
            a.vcodes = st->value_codes;
            a.vscales = st->value_scales;
        }
        a.out = out;
        a.xch = w.xch;
        a.xpart = w.xpart;
        a.xcount = w.xcount;
        a.xepoch = w.xepoch;
        a.status = w.status;
        a.dbg_scores = debug ? debug->scores : nullptr;
        a.dbg_selected = debug ? debug->selected : nullptr;
        a.dbg_exact = debug ? debug->exact_tokens : nullptr;
        a.rescore = debug ? debug->rescore : 0;
        MPA_TRY(launch_unit_decode(p->dtype, Gv, a, Uv, R, s));
        return MPATTN_OK;
    }

    for (int32_t stage = first_stage; stage <= last_stage; ++stage) {
        const char* name = hier ? kHierStages[stage] : kFlatStages[stage];
        const bool attend = name[0] == 'a', merge = name[0] == 'm';
        if (!hier && stage == 0) {
            ScoreArgs a{q, st->key_centroids, Cmax, C, nullptr, nullptr, nullptr, nullptr, 0, nullptr, st->sizes,
                        st->offsets, Cmax + 1, w.s, w.rs, Cmax, nullptr, p->n_q_heads, p->n_kv_heads};
            MPA_TRY(launch_score(p->dtype, G, a, U, s));
        } else if (!hier && stage == 1) {
            SelectArgs se{w.rs, Cmax, nullptr, C, nullptr, token_budget, C, w.selmask, w.Cw, w.sel_ids, w.sel_off,
                          w.sel_pre, Cmax, w.counts, debug ? debug->selected : nullptr, C};
            MPA_TRY(launch_select(se, U, s));
        } else if (hier && stage == 0) {
            ScoreArgs a{q, st->coarse_key_centroids, Dmax, st->n_coarse, nullptr, nullptr, nullptr, nullptr, 0,
                        nullptr, st->coarse_sizes, st->coarse_offsets, Dmax + 1, w.cs, w.crs, Dmax, nullptr,
                        p->n_q_heads, p->n_kv_heads};
            MPA_TRY(launch_score(p->dtype, G, a, U, s));
        } else if (hier && stage == 1) {
            SelectArgs se{w.crs, Dmax, nullptr, st->n_coarse, nullptr, p->coarse_candidate_tokens, st->n_coarse,
                          w.cmask, w.Dw, w.csel_ids, w.csel_off, w.csel_pre, Dmax, w.ccounts,
                          debug ? debug->candidates : nullptr, st->n_coarse};
            MPA_TRY(launch_select(se, U, s));
        } else if (hier && stage == 2) {
            ScoreArgs a{q, st->key_centroids, Cmax, bound, w.ccounts, w.csel_pre, w.csel_off, w.ccounts, Dmax,
                        st->coarse_members, st->sizes, st->offsets, Cmax + 1, w.s, w.rs, Cmax, w.fids,
                        p->n_q_heads, p->n_kv_heads};
            MPA_TRY(launch_score(p->dtype, G, a, U, s));
        } else if (hier && stage == 3) {
            if (debug && debug->selected)
                MPA_TRY(hipMemsetAsync(debug->selected, 0, (size_t)U * C * sizeof(int32_t), s));
            SelectArgs se{w.rs, Cmax, w.fids, bound, w.ccounts, token_budget, C, w.selmask, w.Cw, w.sel_ids,
                          w.sel_off, w.sel_pre, Cmax, w.counts, debug ? debug->selected : nullptr, C};
            MPA_TRY(launch_select(se, U, s));
        } else if (attend) {
            AttendArgs a{};
            a.q = q;
            a.Kx = sorted ? st->sorted_keys : k;
            a.Vx = sorted ? st->sorted_values : v;
            a.token_ids = sorted ? nullptr : st->token_ids;
            a.K = k;
            a.V = v;
            a.sel_off = w.sel_off;
            a.sel_rowpre = w.sel_pre;
            a.sel_stride = Cmax;
            a.counts = w.counts;
            a.Nmax = N;
            a.n_clustered = st->n_clustered;
            a.n_total = n_tokens_total;
            a.sa = SubSrc{w.sel_ids, Cmax, w.counts, w.s, st->sizes, st->value_centroids, Cmax};
            if (hier) {
                a.sb = SubSrc{w.csel_ids, Dmax, w.ccounts, w.cs, st->coarse_sizes, st->coarse_value_centroids, Dmax};
                a.n_sub = want_pseudo ? 2 : 0;
                a.pseudo[0] = PseudoArgs{nullptr, 0, st->n_coarse, nullptr, w.cs, st->coarse_sizes,
                                         st->coarse_value_centroids, Dmax, score_chunks(st->n_coarse)};
                a.pseudo[1] = PseudoArgs{w.fids, Cmax, bound, w.ccounts, w.s, st->sizes, st->value_centroids, Cmax,
                                         score_chunks(bound)};
                a.n_pseudo = want_pseudo ? 2 : 0;
            } else {
                a.n_sub = want_pseudo ? 1 : 0;
                a.pseudo[0] = PseudoArgs{nullptr, 0, C, nullptr, w.s, st->sizes, st->value_centroids, Cmax,
                                         score_chunks(C)};
                a.n_pseudo = want_pseudo ? 1 : 0;
            }
            a.Hq = p->n_q_heads;
            a.Hkv = p->n_kv_heads;
            a.S = S;
            a.part_ml = w.part_ml;
            a.part_acc = w.part_acc;
            a.part_stride = P;
            MPA_TRY(launch_attend(p->dtype, G, a, U, s));
        } else if (merge) {
            MPA_TRY(launch_merge(w.part_ml, w.part_acc, U, G, P, p->n_kv_heads, out, s));
        }
    }
    // optional inspection copies once the selection exists
    if (debug && last_stage >= (hier ? 3 : 1)) {
        if (debug->scores)
            MPA_TRY(hipMemcpy2DAsync(debug->scores, (size_t)C * G * 4, w.s, (size_t)Cmax * G * 4, (size_t)C * G * 4,
                                     U, hipMemcpyDeviceToDevice, s));
        if (debug->exact_tokens)
            MPA_TRY(hipMemcpy2DAsync(debug->exact_tokens, 4, w.counts, 16, 4, U, hipMemcpyDeviceToDevice, s));
    }
    return MPATTN_OK;
}

mpattn_status mpattn_decode(const mpattn_params* p, const void* q, const void* k, const void* v,
                            int32_t n_tokens_total, const mpattn_state* st, int32_t token_budget, int32_t mode,
                            float* out, void* workspace, size_t workspace_bytes, void* stream) {
    const int32_t n = mpattn_decode_stage_count(p);
    if (n == 0) return check_params(p) == MPATTN_OK ? MPATTN_ERR_INVALID_ARG : check_params(p);
    return mpattn_decode_ex(p, q, k, v, n_tokens_total, st, token_budget, mode, out, workspace, workspace_bytes,
                            stream, nullptr, 0, n - 1);
}

mpattn_status mpattn_decode_noalloc(const mpattn_params* p, const void* q, const void* k, const void* v,
                                    int32_t n_tokens_total, const mpattn_state* st, int32_t token_budget,
                                    int32_t mode, float* out, void* stream) {
    const int32_t n = mpattn_decode_stage_count(p);
    if (n == 0) return check_params(p) == MPATTN_OK ? MPATTN_ERR_INVALID_ARG : check_params(p);
    // everything is checked before the first enqueue (the scratch clear)
    mpattn_status rc = check_decode(p, q, k, v, n_tokens_total, st, token_budget, mode, out, 0, n - 1);
    if (rc != MPATTN_OK) return rc;
    if (layout_decode(p, st->capacity_clusters, st->capacity_coarse, nullptr).bytes > kScratchBytes)
        return MPATTN_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((rc = scratch_for(p, st, &ws, (hipStream_t)stream)) != MPATTN_OK) return rc;
    return mpattn_decode_ex(p, q, k, v, n_tokens_total, st, token_budget, mode, out, ws, kScratchBytes, stream,
                            nullptr, 0, n - 1);
}

size_t mpattn_decode_noalloc_max_bytes(void) { return kScratchBytes; }

mpattn_status mpattn_dense_decode(const mpattn_params* p, const void* q, const void* k, const void* v,
                                  int32_t n_tokens, float* out, void* workspace, size_t workspace_bytes,
                                  void* stream) {
    mpattn_status rc = check_params(p);
    if (rc != MPATTN_OK) return rc;
    if (!q || !k || !v || !out) return MPATTN_ERR_INVALID_ARG;
    if (n_tokens < 1 || n_tokens > p->capacity_tokens) return MPATTN_ERR_INVALID_ARG;
    if (p->dtype != MPATTN_BF16) return MPATTN_ERR_UNSUPPORTED;
    const size_t need = dense_ws_bytes(p);
    if (!workspace || workspace_bytes < need) return MPATTN_ERR_WORKSPACE;
    const int U = p->batch * p->n_kv_heads, G = p->n_q_heads / p->n_kv_heads;
    const int S = dense_splits(U);
    float* part_ml = (float*)workspace;
    float* part_acc = (float*)((char*)workspace + align_up((size_t)U * G * S * 2 * 4));
    DenseArgs a{q, k, v, p->capacity_tokens, n_tokens, p->n_q_heads, p->n_kv_heads, part_ml, part_acc};
    const hipStream_t s = (hipStream_t)stream;
    MPA_TRY(launch_dense(G, a, U, S, s));
    MPA_TRY(launch_merge(part_ml, part_acc, U, G, S, p->n_kv_heads, out, s));
    return MPATTN_OK;
}

mpattn_status mpattn_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0) return MPATTN_ERR_INVALID_ARG;
    return hip_status(launch_read_probe(buf, bytes, sink, (hipStream_t)stream));
}

}  // extern "C"
