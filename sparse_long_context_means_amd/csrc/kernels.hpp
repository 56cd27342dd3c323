// kernels.hpp -- host-side launchers of the gfx950 kernels (internal API of
// the library; the public C ABI lives in include/mpattn.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpa {

constexpr int kMaxBlock = 16384;  // largest clustering block (LDS-resident sort)

// Clustering blocks handled by one launch.  Block j (0 <= j < nb) covers
// tokens [p_base + j * block_len, min(p_base + (j + 1) * block_len, n_end))
// and owns clusters starting at c_base + j * cfull; it is seeded as block
// index j_base + j.  Only the last block of a launch may be short.
struct BlockRange {
    int32_t p_base, n_end, c_base, block_len, tpc, cfull, j_base, nb;
};

// Strides shared by all per-unit arrays.
struct UnitGeom {
    int32_t units;  // B * Hkv
    int32_t Nmax;   // token capacity per unit
    int32_t Cmax;   // cluster capacity per unit (rows of the centroid arrays)
};

// ---- clustering (kmeans.hip) --------------------------------------------
hipError_t launch_kmeans_init(int dtype, const void* K, UnitGeom g, BlockRange br, uint64_t seed, float* mu,
                              void* kbar, hipStream_t st);
hipError_t launch_kmeans_assign(int dtype, const void* K, UnitGeom g, BlockRange br, const void* kbar,
                                int32_t* assign, hipStream_t st);
hipError_t launch_kmeans_csr(const int32_t* assign, UnitGeom g, BlockRange br, int32_t* sizes,
                             int32_t* offsets, int32_t* token_ids, hipStream_t st);
// Mean of each cluster's member rows of X for clusters [c_begin, c_begin +
// c_count).  `master` (fp32, may be null) and `store` (storage dtype) receive
// it; an empty cluster is skipped, or zeroed in `store` when empty_zero.
hipError_t launch_segmented_mean(int dtype, const void* X, UnitGeom g, int c_begin, int c_count,
                                 const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids,
                                 float* master, void* store, bool empty_zero, hipStream_t st);
// ---- hierarchical decode in one launch (hier.hip) ------------------------
constexpr int kHierMaxD = 2048;          // coarse clusters per unit
constexpr int kHierMaxF = 4096;          // candidate fine clusters (bounded by the candidate budget)
constexpr int kHierMinReplicas = 3;      // workgroups per unit: at least 3, so a share fits ...
constexpr int kHierMaxReplicas = 8;
constexpr int kHierMaxShare = (kHierMaxD + kHierMinReplicas - 1) / kHierMinReplicas +
                              (kHierMaxF + kHierMinReplicas - 1) / kHierMinReplicas + 16;  // ... in LDS

struct HierArgs {
    const void* q;               // [B][Hq][d]
    const void* kbar;            // fine [U][Cmax][d]
    const void* vbar;
    const int32_t* sizes;        // fine [U][Cmax]
    const int32_t* offsets;      // fine [U][Cmax + 1]
    const void* Kx;              // exact rows: sorted copy, or K, V gathered through token_ids
    const void* Vx;
    const int32_t* token_ids;    // null when Kx, Vx are the sorted copy
    const void* K;               // tail rows
    const void* V;
    const void* ckbar;           // coarse [U][Dmax][d]
    const void* cvbar;
    const int32_t* csizes;       // coarse [U][Dmax]
    const int32_t* coffsets;     // coarse [U][Dmax + 1]: start in cmembers
    const int32_t* cmembers;     // [U][Cmax]
    int32_t Cmax, Dmax, C, D, Nmax, n_clustered, n_total, budget, cand_budget;
    int32_t pseudo;
    int32_t Hq, Hkv;
    float* out;                  // [B][Hq][d]
    uint64_t* xch;               // [U][R][Dmax] tagged coarse-key words, slot r read by workgroup r
    uint64_t* xpart;             // [U][R][G][d + 2] tagged partial words
    uint64_t* xcount;            // [U] arrival counters, 0 between decodes (the merging workgroup resets)
    uint32_t* xepoch;            // [U] tag of the unit's last decode (the merging workgroup writes it)
    uint32_t* status;            // [2] counters: key-exchange fallbacks, partial words given up on
    int32_t* dbg_selected;       // optional [U][C]
    int32_t* dbg_candidates;     // optional [U][D]
    int32_t* dbg_exact;          // optional [U]
    int32_t rescore;             // 0; 1: every workgroup scores all coarse clusters; 2: as if no key came
};
int hier_replicas(int units);
bool hier_path_fits(int dtype, int G, int max_coarse, int cand_budget);
hipError_t launch_hier_decode(int dtype, int G, const HierArgs& a, int units, int replicas, hipStream_t st);

// fp8 copies of centroid rows [c_begin, c_begin + c_count) of every unit (codes.hip)
hipError_t launch_encode_codes(UnitGeom g, int c_begin, int c_count, const void* kbar, const void* vbar,
                               uint8_t* kcodes, uint8_t* kscales, uint8_t* vcodes, uint8_t* vscales, hipStream_t st);
hipError_t launch_sorted_copy(int dtype, const void* K, const void* V, UnitGeom g, int p_begin, int count,
                              const int32_t* token_ids, void* SK, void* SV, hipStream_t st);

// Coarse level: size-weighted k-means over each block's non-empty fine key
// centroids.  `fine` describes the fine blocks (token ranges and cluster
// ranges); coarse block j owns coarse clusters from d_base + j * dfull and has
// ceil(L_j / coarse_tpc) of them.
struct CoarseRange {
    BlockRange fine;
    int32_t d_base, coarse_tpc, dfull, Dmax;
};
hipError_t launch_coarse_build(int dtype, UnitGeom g, CoarseRange cr, uint64_t seed, int iters,
                               const void* kbar, const void* vbar, const int32_t* sizes, float* cmu,
                               void* ckbar, void* cvbar, int32_t* csizes, int32_t* parent, int32_t* coffsets,
                               int32_t* cmembers, hipStream_t st);

// ---- decode (decode.hip) --------------------------------------------------
struct ScoreArgs {
    const void* q;               // [B][Hq][d]
    const void* cent;            // [U][cent_rows][d] key centroids
    int32_t cent_rows;
    int32_t n_items;             // items per unit (host bound)
    const int32_t* n_items_dev;  // optional per-unit count: n_items_dev[unit * 4]
    // optional item source: the member rows of a selection (list_pre/list_off
    // of a previous select, count list_counts[unit * 4 + 1]), mapped through
    // members[] to cluster ids
    const int32_t* list_pre;     // [U][list_stride + 1]
    const int32_t* list_off;     // [U][list_stride]
    const int32_t* list_counts;  // [U][4]
    int32_t list_stride;
    const int32_t* members;      // [U][cent_rows] position -> cluster id
    const int32_t* sizes;        // [U][cent_rows] cluster sizes (budget weights)
    const int32_t* offsets;      // [U][off_stride] member start by cluster id (CSR)
    int32_t off_stride;
    float* s_out;                // [U][cent_rows][G] scores by cluster id
    int4* rs_out;                // [U][rs_stride] (key bits, weight, first member, member rows) by item
    int32_t rs_stride;
    int32_t* ids_out;            // optional [U][rs_stride]: cluster id of each item
    int32_t Hq, Hkv;
};
// Workgroups (chunks) of a score launch over n_items items.
int score_chunks(int n_items);
hipError_t launch_score(int dtype, int G, const ScoreArgs& a, int units, hipStream_t st);

struct SelectArgs {
    const int4* rs;              // [U][rs_stride] records of the score pass
    int32_t rs_stride;
    const int32_t* ids;          // optional [U][rs_stride]: cluster id per item (else id = item)
    int32_t n_items;             // host count (bound when n_items_dev is set)
    const int32_t* n_items_dev;  // optional per-unit count at n_items_dev[unit * 4]
    int32_t budget;
    int32_t mask_bits;           // cluster ids < mask_bits
    uint32_t* selmask;           // [U][mask_stride] 1 bit per cluster id: selected
    int32_t mask_stride;
    int32_t* sel_ids;            // [U][sel_stride] selected cluster ids, item order
    int32_t* sel_off;            // [U][sel_stride] their first member position
    int32_t* sel_rowpre;         // [U][sel_stride + 1] exclusive prefix of member rows
    int32_t sel_stride;
    int32_t* counts;             // [U][4]: member rows, selected items, 0, 0
    int32_t* dbg_selected;       // optional [U][dbg_stride] by cluster id
    int32_t dbg_stride;
};
// Approximate term of every non-empty item, streamed by the attend launch in
// chunks of 256 items.
struct PseudoArgs {
    const int32_t* ids;          // optional [U][ids_stride]: cluster id per item
    int32_t ids_stride;
    int32_t n_items;             // host count (bound when n_items_dev is set)
    const int32_t* n_items_dev;  // optional per-unit count at n_items_dev[unit * 4]
    const float* s;              // [U][rows][G] scores by cluster id
    const int32_t* sizes;        // [U][rows]
    const void* vbar;            // [U][rows][d]
    int32_t rows;
    int32_t chunks;              // score_chunks(n_items)
};
// Budget cut of every unit (one workgroup each).
hipError_t launch_select(const SelectArgs& a, int units, hipStream_t st);

// Selected clusters whose approximate term the score pass added and attend
// removes again.
struct SubSrc {
    const int32_t* ids;          // [U][ids_stride] selected cluster ids
    int32_t ids_stride;
    const int32_t* counts;       // count at counts[unit * 4 + 1]
    const float* s;              // [U][rows][G] scores
    const int32_t* sizes;        // [U][rows]
    const void* vbar;            // [U][rows][d]
    int32_t rows;
};
struct AttendArgs {
    const void* q;
    const void* Kx;              // exact-row source: sorted copy or K
    const void* Vx;
    const int32_t* token_ids;    // non-null: member positions go through token ids
    const void* K;               // tail rows
    const void* V;
    const int32_t* sel_off;      // [U][sel_stride]
    const int32_t* sel_rowpre;   // [U][sel_stride + 1]
    int32_t sel_stride;
    const int32_t* counts;       // [U][4] of the (fine) select
    int32_t Nmax;
    int32_t n_clustered, n_total;
    int32_t n_sub;               // lists removed (0, 1 or 2)
    SubSrc sa, sb;
    int32_t Hq, Hkv, S;
    int32_t n_pseudo;            // approximate-term sources, spread over the splits (0 .. 2)
    PseudoArgs pseudo[2];
    float* part_ml;              // [U][G][part_stride][2], slots 0 .. S-1
    float* part_acc;             // [U][G][part_stride][d]
    int32_t part_stride;
};
hipError_t launch_attend(int dtype, int G, const AttendArgs& a, int units, hipStream_t st);
// Merges the P partial slots of every (unit, query head).
hipError_t launch_merge(const float* part_ml, const float* part_acc, int units, int G, int P, int Hkv,
                        float* out, hipStream_t st);

// ---- whole decode step per unit (unit.hip) ---------------------------------
struct UnitArgs {
    const void* q;               // [B][Hq][d]
    const void* kbar;            // [U][Cmax][d]
    const void* vbar;            // [U][Cmax][d]
    const int32_t* sizes;        // [U][Cmax]
    const int32_t* offsets;      // [U][Cmax + 1]
    const void* Kx;              // exact-row source: sorted copy or K
    const void* Vx;
    const int32_t* token_ids;    // non-null: member positions go through token ids
    const void* K;               // tail rows
    const void* V;
    int32_t Cmax, C, Nmax, n_clustered, n_total, budget;
    int32_t pseudo;              // 1: approximate unselected clusters; 0: omit them
    int32_t Hq, Hkv;             // Hkv: units per sequence
    int32_t ugroup;              // units per state unit (1; G when each query head is its own unit)
    // fp8 copies of the centroids ([U][Cmax][d] codes, [U][Cmax][d / 32]
    // scale bytes); when kcodes is set they replace kbar and vbar
    const uint8_t* kcodes;
    const uint8_t* kscales;
    const uint8_t* vcodes;
    const uint8_t* vscales;
    float* out;                  // [B][Hq][d]
    // replica exchange (several replicas): words are (tag << 32 | 32-bit value)
    uint64_t* xch;               // [U][R][Cmax]: keys, slot r read by replica r
    uint64_t* xpart;             // [U][R][G][d + 2]: partial sums, m, l of each replica
    uint64_t* xcount;            // [U]: replicas counted in, 0 between decodes (the merging replica resets)
    uint32_t* xepoch;            // [U]: tag of the unit's last decode; this call's is one more (never 0)
    uint32_t* status;            // [2]: key-exchange fallbacks, partial words given up on
    int32_t rescore;             // 1: every workgroup scores every cluster; 2: one wave does, as after a timeout
    float* dbg_scores;           // optional [U][C][G]
    int32_t* dbg_selected;       // optional [U][C]
    int32_t* dbg_exact;          // optional [U]
};
// Replicas (workgroups per unit) of the per-unit path for C clusters: one when
// C <= 2048 and there are at least 256 units, else at least two, shares of
// <= 1024 clusters and at least 256 workgroups in all (up to 8 per unit).
int unit_replicas(int n_clusters, int units);
// Whether the per-unit path supports this storage dtype, group size and
// cluster capacity.
bool unit_path_fits(int dtype, int G, int cmax);
hipError_t launch_unit_decode(int dtype, int G, const UnitArgs& a, int units, int replicas, hipStream_t st);

// ---- dense decode (dense.hip) ----------------------------------------------
struct DenseArgs {
    const void* q;               // [B][Hq][d] bf16
    const void* K;               // [U][Nmax][d] bf16
    const void* V;
    int32_t Nmax, n_tokens, Hq, Hkv;
    float* part_ml;              // [U][G][S][2]
    float* part_acc;             // [U][G][S][d]
};
// Token splits of the dense decode for this many units.
int dense_splits(int units);
hipError_t launch_dense(int G, const DenseArgs& a, int units, int splits, hipStream_t st);

// ---- measurement (probe.hip) ----------------------------------------------
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t st);

}  // namespace mpa
