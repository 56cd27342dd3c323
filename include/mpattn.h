/*
 * mpattn.h -- C ABI of the Multipole Attention decode path on AMD gfx950.
 *
 * The method (web pages on "Multipole Attention for Efficient Long Context
 * Reasoning", arXiv 2506.13059):
 *   - mlsanity.com paper page, "Abstract (arXiv)": keys are grouped by
 *     clustering; the centroids both pick the important keys, which get exact
 *     attention, and stand in for the remaining keys; a fast update re-clusters
 *     newly generated tokens.
 *   - atlas.scime.ai summary, "Approach": centroid scores select keys for exact
 *     attention and the unselected clusters contribute through their value
 *     centroids; a hierarchical variant and a blockwise sliding-window online
 *     update exist.
 *   - atlas.scime.ai summary, "Measured effects reported in the paper": one
 *     centroid per 16 tokens and clustering blocks of a few thousand tokens are
 *     the defaults.
 * The approximate term of an unselected cluster c is n_c * exp(q . Kbar_c /
 * sqrt(d)) applied to its value centroid Vbar_c, in the numerator and in the
 * softmax denominator.
 *
 * Conventions shared by every entry point
 *   - Pointers marked "device" are HIP device addresses; all other pointers
 *     are host addresses.  Every buffer is allocated and owned by the caller;
 *     the library allocates nothing and is re-entrant on distinct states and
 *     workspaces.
 *   - Layouts are dense and row-major.  K and V are [B][Hkv][capacity_tokens][d]
 *     (capacity_tokens rows per (sequence, KV head) "unit"), q is [B][Hq][d],
 *     out is [B][Hq][d] float32.  Query head hq belongs to KV head hq / G with
 *     G = Hq / Hkv.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it in stream order; no call waits for the device.  The host
 *     counters in mpattn_state are updated when the work is enqueued.
 *   - Every argument is validated before anything is enqueued; on an error
 *     nothing is enqueued and a negative status is returned.  A launch failure
 *     reported by the HIP runtime after enqueueing maps to MPATTN_ERR_HIP.
 *   - Results are deterministic: the same inputs give the same bits.
 *   - The library keeps no global state: a decode's per-call tags live in
 *     its workspace.
 */
#ifndef MPATTN_H
#define MPATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MPATTN_OK = 0,
    MPATTN_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shape */
    MPATTN_ERR_UNSUPPORTED = -2, /* valid but not implemented (head_dim != 128, G > 8, ...) */
    MPATTN_ERR_WORKSPACE = -3,   /* workspace missing or smaller than mpattn_workspace_bytes */
    MPATTN_ERR_CAPACITY = -4,    /* tokens or clusters beyond the state's capacity */
    MPATTN_ERR_HIP = -5          /* the HIP runtime reported a launch error */
} mpattn_status;

typedef enum { MPATTN_F32 = 0, MPATTN_BF16 = 1 } mpattn_dtype;

/* What the decode reads for the clusters' key and value centroids.  The
 * pages keep the centroids in the cache's own precision; the fp8 format is
 * a bandwidth option of this library (the centroids are over half of the
 * bytes a decode step at 95% sparsity reads):
 *   MPATTN_CENTROIDS_STORED: the stored centroids (dtype);
 *   MPATTN_CENTROIDS_FP8: fp8 copies that the build and update write next
 *     to the stored centroids: every run of 32 values of a centroid row
 *     shares a scale 2^E, E the least integer >= -126 with
 *     max|x| * 2^-E <= 448, stored as the byte E + 127; each value is the
 *     E4M3 code (OCP 8-bit floating point: bias 7, 3 mantissa bits,
 *     subnormals, largest finite 448) nearest to x * 2^-E, ties to the even
 *     code, sign bit copied from x.  The decode computes with the decoded
 *     values code * 2^E.  bf16 storage, flat method, one-launch decode
 *     only.  The k-means itself always uses the stored centroids. */
typedef enum { MPATTN_CENTROIDS_STORED = 0, MPATTN_CENTROIDS_FP8 = 1 } mpattn_centroid_format;

typedef enum { MPATTN_OP_BUILD = 0, MPATTN_OP_UPDATE = 1, MPATTN_OP_DECODE = 2, MPATTN_OP_DENSE = 3 } mpattn_op;

typedef enum {
    MPATTN_MODE_MULTIPOLE = 0, /* unselected clusters approximated by their value centroids */
    MPATTN_MODE_OMIT = 1,      /* unselected clusters dropped (the ablation the pages compare with) */
    MPATTN_MODE_PER_HEAD = 2   /* as MULTIPOLE, but every query head ranks and cuts on its own scores */
} mpattn_mode;

/* Shape and method parameters (host struct, read-only for the library). */
typedef struct mpattn_params {
    int32_t batch;                      /* B >= 1 */
    int32_t n_q_heads;                  /* Hq, a multiple of Hkv */
    int32_t n_kv_heads;                 /* Hkv >= 1; G = Hq / Hkv must be 1, 2, 4 or 8 */
    int32_t head_dim;                   /* d; must be 128 */
    int32_t dtype;                      /* mpattn_dtype of K, V, q and the stored centroids */
    int32_t capacity_tokens;            /* rows per unit in K, V and the token arrays of the state */
    int32_t tokens_per_centroid;        /* r: a block of L tokens gets ceil(L / r) clusters (default 16) */
    int32_t cluster_block;              /* tokens per clustering block, 1 .. 16384 (default 8192) */
    int32_t build_iters;                /* Lloyd rounds of mpattn_build_clusters, >= 1 (default 10) */
    int32_t update_iters;               /* Lloyd rounds per block of mpattn_update_window, >= 1 (default 5) */
    int32_t coarse_tokens_per_centroid; /* 0: flat method; else a block of L tokens gets
                                           ceil(L / this) coarse clusters (default 128) */
    int32_t coarse_iters;               /* weighted Lloyd rounds of the coarse level, >= 1 (default 10) */
    int32_t coarse_candidate_tokens;    /* hierarchical decode: token budget of the coarse candidates */
    int32_t splits;                     /* decode work splits per unit; 0 = chosen by the library
                                           (> 0 also selects the split launches of the flat method) */
    int32_t centroid_format;            /* an mpattn_centroid_format value; default STORED */
    uint64_t seed;                      /* seeds the k-means initialisation */
} mpattn_params;

/*
 * Cluster state of all units (caller-owned device arrays + host counters).
 * Cmax = capacity_clusters, Dmax = capacity_coarse, Nmax = capacity_tokens.
 * Clusters of a unit are numbered in block order; block j's tokens occupy
 * token_ids positions equal to its own token range, ordered by
 * (cluster, token).
 */
typedef struct mpattn_state {
    void* key_centroids;      /* device [B][Hkv][Cmax][d] dtype: stored key centroids          */
    void* value_centroids;    /* device [B][Hkv][Cmax][d] dtype: stored value centroids        */
    float* key_centroids_f32; /* device [B][Hkv][Cmax][d]: unrounded key-centroid means         */
    int32_t* sizes;           /* device [B][Hkv][Cmax]: member count of each cluster          */
    int32_t* offsets;         /* device [B][Hkv][Cmax+1]: start of each cluster in token_ids   */
    int32_t* token_ids;       /* device [B][Hkv][Nmax]: member token ids                       */
    int32_t* assign;          /* device [B][Hkv][Nmax]: cluster id of each clustered token      */
    void* sorted_keys;        /* optional device [B][Hkv][Nmax][d]: K rows in token_ids order   */
    void* sorted_values;      /* optional device [B][Hkv][Nmax][d]: V rows in token_ids order;
                                 both sorted arrays or neither.  When present, the build and
                                 update fill them and the decode reads exact rows from them
                                 (contiguous per cluster) instead of gathering by token id.   */
    /* coarse level of the hierarchy; all NULL for the flat method */
    void* coarse_key_centroids;      /* device [B][Hkv][Dmax][d] dtype */
    void* coarse_value_centroids;    /* device [B][Hkv][Dmax][d] dtype */
    float* coarse_key_centroids_f32; /* device [B][Hkv][Dmax][d] */
    int32_t* coarse_sizes;           /* device [B][Hkv][Dmax]: member tokens of each coarse cluster */
    int32_t* coarse_offsets;         /* device [B][Hkv][Dmax+1]: start in coarse_members          */
    int32_t* coarse_members;         /* device [B][Hkv][Cmax]: non-empty fine ids by (coarse, fine);
                                        the blocks' lists follow each other */
    int32_t* parent;                 /* device [B][Hkv][Cmax]: coarse id of each fine cluster, -1 if empty */
    /* fp8 copies of the centroids (MPATTN_CENTROIDS_FP8; else may be NULL) */
    uint8_t* key_codes;              /* device [B][Hkv][Cmax][d]: E4M3 codes of key_centroids        */
    uint8_t* key_scales;             /* device [B][Hkv][Cmax][d / 32]: scale bytes E + 127            */
    uint8_t* value_codes;            /* device [B][Hkv][Cmax][d]: E4M3 codes of value_centroids      */
    uint8_t* value_scales;           /* device [B][Hkv][Cmax][d / 32] */
    int32_t capacity_clusters;       /* Cmax >= mpattn_max_clusters(params) is always enough */
    int32_t capacity_coarse;         /* Dmax (0 for the flat method) */
    /* host counters, identical for every unit; set to 0 before the first build */
    int32_t n_clustered;             /* tokens [0, n_clustered) are clustered */
    int32_t n_clusters;              /* clusters in use per unit */
    int32_t n_coarse;                /* coarse clusters in use per unit */
    int32_t n_blocks;                /* clustering blocks so far (seeds the next block) */
} mpattn_state;

/* Optional per-call outputs of the decode, for inspection and tests.
 * Any field may be NULL. */
typedef struct mpattn_decode_debug {
    float* scores;          /* device [B][Hkv][n_clusters][G]: q . Kbar_c / sqrt(d) (fine level) */
    int32_t* selected;      /* device [B][Hkv][n_clusters]: 1 for clusters attended exactly      */
    int32_t* candidates;    /* device [B][Hkv][n_coarse]: 1 for coarse candidates (hierarchical) */
    int32_t* exact_tokens;  /* device [B][Hkv]: tokens of the selected clusters                   */
    int32_t rescore;        /* one-launch decodes only (flat: all clusters; hierarchical: the
                               coarse clusters); 0: normal.  1: every workgroup of a unit scores
                               all of them instead of taking the other workgroups' keys.  2: as if
                               those keys never arrived (the path taken when a workgroup is late:
                               it scores them itself).  The result is the same bits in all three
                               cases. */
} mpattn_decode_debug;

/* Human-readable text of a status code (static storage); any int is accepted
 * ("unknown status" for a value that is not an mpattn_status). */
const char* mpattn_status_string(int32_t status);

/* Clusters per unit that any build/update sequence within capacity_tokens can
 * need: ceil(N / r) + ceil(N / cluster_block) + 1 for N = capacity_tokens.
 * Returns 0 when the parameters are invalid. */
int32_t mpattn_max_clusters(const mpattn_params* params);

/* Same bound for the coarse level (0 for the flat method). */
int32_t mpattn_max_coarse(const mpattn_params* params);

/* Workspace bytes an operation needs for a state of `capacity_clusters`
 * clusters (and `capacity_coarse` coarse clusters).  0 means no workspace.
 * Returns (size_t)-1 when the parameters are invalid.  Decodes that share a
 * workspace must not overlap in time.  A decode workspace must hold zeros
 * before its first decode, and again before it serves other parameters or
 * capacities, and must not be written by anything else between decodes: the
 * workgroups of a unit exchange tagged words and count themselves in on a
 * counter through it; it keeps the tag of each unit's last decode and every
 * counter back at zero (a decode leaves it valid for the next one).
 * Its first 8 bytes are two uint32 counters that the one-launch decodes add
 * to and never reset:
 *   [0] workgroups that scored the other workgroups' clusters themselves
 *       because those ranking keys had not arrived within a bounded wait
 *       (the same bits result, later; debug rescore 2 forces this path);
 *   [1] output values written as NaN because another workgroup's partial sum
 *       had not arrived within a bounded wait (a failure to check for). */
size_t mpattn_workspace_bytes(const mpattn_params* params, int32_t capacity_clusters, int32_t capacity_coarse,
                              int32_t op);

/*
 * Build: cluster tokens [0, n_tokens) of every unit from scratch (pages: keys
 * grouped by k-means ahead of decoding; "blockwise" clustering).  Blocks of
 * cluster_block tokens (the last may be shorter) are clustered independently:
 * ceil(L / r) centroids per block, seeded with distinct tokens of the block
 * chosen by a splitmix64 stream keyed by (seed, unit, block), then build_iters
 * Lloyd rounds (nearest centroid by squared Euclidean distance on bf16/fp32
 * keys with fp32 accumulation, ties to the lowest cluster id; mean update; an
 * empty cluster keeps its centroid).  Value centroids are member means of V.
 * With coarse_tokens_per_centroid > 0 the coarse level is built as well.
 *   k, v : device K and V; rows [0, n_tokens) of each unit are read.
 *   state: device arrays written; counters reset and set (n_clustered =
 *          n_tokens, n_blocks = ceil(n_tokens / cluster_block)).
 * Errors: INVALID_ARG, UNSUPPORTED, CAPACITY (n_tokens > capacity_tokens or
 * clusters > capacity_clusters), WORKSPACE, HIP.
 */
mpattn_status mpattn_build_clusters(const mpattn_params* params, const void* k, const void* v,
                                    int32_t n_tokens, mpattn_state* state, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * Online update (pages: "fast cluster update" of generated tokens;
 * "blockwise sliding-window" update).  Tokens [n_clustered, n_tokens_total)
 * form an unclustered tail that the decode attends exactly.  While the tail
 * holds at least cluster_block tokens, its first cluster_block tokens are
 * clustered as a new block (update_iters rounds, same seeding rule with the
 * next block index) and their clusters are appended; n_clustered advances by
 * cluster_block.  Calling it with a shorter tail enqueues nothing.
 * Errors: as mpattn_build_clusters; INVALID_ARG if n_tokens_total <
 * n_clustered.
 */
mpattn_status mpattn_update_window(const mpattn_params* params, const void* k, const void* v,
                                   int32_t n_tokens_total, mpattn_state* state, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * Decode step (pages: exact attention on the top-scoring clusters, centroid
 * terms for the rest).  For every unit and each of its G query heads:
 * s_c = q . Kbar_c / sqrt(d) for non-empty clusters; the unit ranks clusters by
 * the mean of s_c over its G heads (ties by lower id) and selects the longest
 * prefix whose sizes sum to at most token_budget.  Output per query head:
 *   out = (sum_exact e^{l_i} v_i + sum_unselected n_c e^{s_c} Vbar_c)
 *       / (sum_exact e^{l_i}     + sum_unselected n_c e^{s_c})
 * where the exact set is every token of a selected cluster plus the
 * unclustered tail [n_clustered, n_tokens_total).  MPATTN_MODE_OMIT drops the
 * unselected terms.  MPATTN_MODE_PER_HEAD is the alternative to the shared
 * selection (the pages do not say who selects under grouped-query attention):
 * each query head ranks the clusters of its KV head by its own s_c and takes
 * its own cut under token_budget, so one KV head may read up to G different
 * exact sets; it runs on the one-launch path only (UNSUPPORTED elsewhere), and
 * its inspection outputs are per query head ([B][Hq][C] selected, [B][Hq]
 * exact_tokens, [B][Hq][C] scores).  The hierarchical method (coarse level present) first
 * selects coarse candidates under coarse_candidate_tokens, then selects fine
 * clusters inside them; unselected fine clusters of candidates and all
 * non-candidate coarse clusters give the approximate terms.  Both cuts break
 * equal keys by the lower cluster id (coarse id, then fine id), whatever
 * order the candidates' fine clusters are listed in.
 *   q   : device [B][Hq][d] dtype.      k, v: device K, V (tail rows, and all
 *   exact rows when the state has no sorted copy).   out: device [B][Hq][d] fp32.
 *   token_budget >= 0 tokens per unit.
 * Errors: INVALID_ARG (null, n_tokens_total < n_clustered or > capacity,
 * negative budget, no clusters), UNSUPPORTED, WORKSPACE, HIP.
 */
mpattn_status mpattn_decode(const mpattn_params* params, const void* q, const void* k, const void* v,
                            int32_t n_tokens_total, const mpattn_state* state, int32_t token_budget,
                            int32_t mode, float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * mpattn_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same decode, with the library's own workspace -- a file-scope device
 * array of mpattn_decode_noalloc_max_bytes() bytes that every GPU the library
 * runs on holds until the process ends.  It allocates nothing.  The array is
 * cleared on its first use on a device and whenever the decode layout
 * (parameters and capacities) differs from the previous call's on that
 * device; otherwise it keeps the previous call's contents (call tags, and
 * the two counters described under mpattn_workspace_bytes, which this entry
 * point gives no access to).  All calls on one GPU share the array: calls
 * that overlap in time on one GPU race, so the caller serialises them (one
 * stream, or events).
 *   Arguments as mpattn_decode without the workspace.
 * Errors: as mpattn_decode; MPATTN_ERR_WORKSPACE when the layout needs more
 * than mpattn_decode_noalloc_max_bytes() (checked, with every other argument,
 * before anything is enqueued); MPATTN_ERR_UNSUPPORTED for a device index of
 * 64 or more.
 */
mpattn_status mpattn_decode_noalloc(const mpattn_params* params, const void* q, const void* k, const void* v,
                                    int32_t n_tokens_total, const mpattn_state* state, int32_t token_budget,
                                    int32_t mode, float* out, void* stream);

/* Size of the device array mpattn_decode_noalloc uses as its workspace. */
size_t mpattn_decode_noalloc_max_bytes(void);

/*
 * Dense decode: exact attention of every query head over all tokens
 * [0, n_tokens) of its KV head, the comparison point of the sparse decode
 * (pages: atlas summary, "Key results": the speedups are quoted against a
 * split-K dense decode).  out[b][hq] = sum_i e^{l_i} v_i / sum_i e^{l_i} with
 * l_i = q_hq . k_i / sqrt(d).  The tokens are split into ranges processed in
 * parallel, then merged (log-sum-exp).  bf16 storage only.
 *   q: device [B][Hq][d]; k, v: device [B][Hkv][capacity_tokens][d];
 *   out: device [B][Hq][d] fp32.  workspace: mpattn_workspace_bytes(...,
 *   MPATTN_OP_DENSE) bytes, no initial contents needed.
 * Errors: INVALID_ARG (null, n_tokens < 1 or > capacity_tokens), UNSUPPORTED
 * (fp32 storage), WORKSPACE, HIP.
 */
mpattn_status mpattn_dense_decode(const mpattn_params* params, const void* q, const void* k, const void* v,
                                  int32_t n_tokens, float* out, void* workspace, size_t workspace_bytes,
                                  void* stream);

/* Number of kernel stages one decode enqueues (for timing stage by stage):
 * for the hierarchical method 1 (hier_unit) when the whole step of a unit
 * runs in one launch -- bf16 storage, splits = 0, groups of 1, 2 or 4 query
 * heads, mpattn_max_coarse <= 2048 and coarse_candidate_tokens <= 4096 --
 * else 6 (coarse_score, coarse_select, fine_score, fine_select, attend,
 * merge); for the flat method 1 (unit) when the whole step of a unit runs in
 * one launch -- bf16 storage, splits = 0, at least 16 units and at most 4096
 * clusters per unit -- else 4 (score, select, attend, merge).  The forms of a
 * method compute the same cuts and, up to fp32 summation order, the same
 * output. */
int32_t mpattn_decode_stage_count(const mpattn_params* params);

/* Name of decode stage i (static storage), NULL if out of range. */
const char* mpattn_decode_stage_name(const mpattn_params* params, int32_t stage);

/*
 * mpattn_decode with optional inspection outputs and a stage range: enqueues
 * decode stages [first_stage, last_stage] only.  Intermediate results stay in
 * the workspace, so consecutive calls covering 0 .. count-1 with the same
 * arguments equal one mpattn_decode.  debug may be NULL.
 */
mpattn_status mpattn_decode_ex(const mpattn_params* params, const void* q, const void* k, const void* v,
                               int32_t n_tokens_total, const mpattn_state* state, int32_t token_budget,
                               int32_t mode, float* out, void* workspace, size_t workspace_bytes,
                               void* stream, const mpattn_decode_debug* debug, int32_t first_stage,
                               int32_t last_stage);

/*
 * Measurement utility: streams `bytes` (a multiple of 16) from the device
 * buffer `buf` with 16-byte loads and no reuse, so that the achievable HBM
 * read rate can be timed next to the decode.  `sink` (device, one uint32) is
 * written only if the XOR of all data equals an arbitrary constant.
 * Errors: INVALID_ARG (null pointer, bad size), HIP.
 */
mpattn_status mpattn_read_probe(const void* buf, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MPATTN_H */
