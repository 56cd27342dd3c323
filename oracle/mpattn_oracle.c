/*
 * mpattn_oracle.c -- plain, slow, fp64 CPU statement of the Multipole Attention
 * decode path.  TEST INFRASTRUCTURE ONLY: the test-suite, the package's smoke
 * check and the benchmark's CPU-baseline leg are the only code allowed to load
 * it.  It shares no source, header, table or helper with the GPU library and
 * must never sit on the product path.
 *
 * Sources (web pages on "Multipole Attention for Efficient Long Context
 * Reasoning", arXiv 2506.13059):
 *   [ABS]  mlsanity.com paper page, section "Abstract (arXiv)": keys are
 *          clustered, centroids pick the important keys and approximate the
 *          rest; a fast update re-clusters generated tokens.
 *   [APP]  atlas.scime.ai summary, section "Approach": centroid scores select
 *          keys for exact attention; unselected clusters are approximated with
 *          value centroids; blockwise sliding-window online update; a
 *          hierarchical variant.
 *   [SUM]  atlas.scime.ai summary, opening sentence: exact attention on the
 *          top-scoring clusters, centroid attention for the rest.
 *   [ABL]  atlas.scime.ai summary, table "Measured effects reported in the
 *          paper": 1 centroid per 16 tokens and clustering blocks between 4K
 *          and 16K tokens are the defaults the ablations move away from.
 *   [HOM]  colemanhooper.org: K-means over the keys ahead of inference; the
 *          query is compared with the key centroids to find important keys.
 * Steps the pages leave open are fixed by readings that are stated at each
 * function and listed with the design notes of the repository.
 *
 * Every floating-point step is computed in double precision.  "Storage"
 * rounding models the dtype the centroids are kept in (exact, binary32 or
 * bfloat16); it is applied exactly where the method stores a centroid.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_EXACT 0
#define ORC_F32 1
#define ORC_BF16 2

/* ------------------------------------------------------------------------- */
/* Rounding to the storage dtype (round to nearest, ties to even).           */
/* ------------------------------------------------------------------------- */

/* bfloat16 keeps 8 significant bits and the binary32 exponent range.  The
 * rounding is done from the double directly (no detour through binary32). */
static double round_bf16(double x) {
    if (x == 0.0 || !isfinite(x)) return x;
    int e;
    double m = frexp(x, &e);           /* x = m * 2^e, 0.5 <= |m| < 1      */
    double y;
    if (e - 1 < -126) {                /* below the normal range: fixed quantum 2^-133 */
        double quantum = ldexp(1.0, -133);
        y = nearbyint(x / quantum) * quantum;
    } else {
        y = ldexp(nearbyint(ldexp(m, 8)), e - 8);   /* nearbyint rounds ties to even */
    }
    if (fabs(y) > 3.3895313892515355e+38) return copysign(INFINITY, x);
    return y;
}

double orc_round_storage(double x, int storage) {
    if (storage == ORC_EXACT) return x;
    if (storage == ORC_F32) return (double)(float)x;   /* C conversion: nearest, ties to even */
    return round_bf16(x);
}

void orc_round_array(const double* x, int64_t n, int storage, double* y) {
    for (int64_t i = 0; i < n; ++i) y[i] = orc_round_storage(x[i], storage);
}

/* ------------------------------------------------------------------------- */
/* Seeded initialisation: splitmix64 (Steele, Lea & Flood, "Fast splittable  */
/* pseudorandom number generators", OOPSLA 2014) used as a counter-based     */
/* generator, and a partial Fisher-Yates shuffle (Durstenfeld form).          */
/* The pages only say the k-means is seeded; which tokens seed it is a        */
/* reading: C distinct tokens of the block drawn uniformly.                   */
/* ------------------------------------------------------------------------- */

static const uint64_t SM64_GAMMA = 0x9E3779B97F4A7C15ull;

uint64_t orc_sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Draw t (t = 0, 1, ...) of the stream whose state starts at s0: the value the
 * sequential generator returns on its (t+1)-th call. */
uint64_t orc_sm64_draw(uint64_t s0, uint64_t t) {
    return orc_sm64_mix(s0 + (t + 1) * SM64_GAMMA);
}

/* Start state of the stream that seeds clustering block `block` of unit
 * `unit` (unit = b * n_kv_heads + h).  `level` is 0 for the token-level
 * clustering and 1 for the coarse level of the hierarchy. */
uint64_t orc_block_stream(uint64_t seed, int64_t unit, int64_t block, int level) {
    uint64_t key = ((uint64_t)unit << 32) + (uint64_t)block + ((uint64_t)level << 62);
    return seed ^ orc_sm64_mix(key);
}

/* The first `count` entries of a partial Fisher-Yates shuffle of [0, n):
 * step t swaps position t with t + (draw_t mod (n - t)). */
int orc_init_indices(uint64_t s0, int32_t n, int32_t count, int32_t* out) {
    if (count > n || n <= 0) return -1;
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)n);
    if (!perm) return -2;
    for (int32_t i = 0; i < n; ++i) perm[i] = i;
    for (int32_t t = 0; t < count; ++t) {
        uint64_t x = orc_sm64_draw(s0, (uint64_t)t);
        int32_t r = t + (int32_t)(x % (uint64_t)(n - t));
        int32_t tmp = perm[t];
        perm[t] = perm[r];
        perm[r] = tmp;
        out[t] = perm[t];
    }
    free(perm);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Lloyd's k-means, one step at a time ([ABS], [HOM]: keys grouped by        */
/* K-means).  Distance: squared Euclidean on the cached key vectors.          */
/* ------------------------------------------------------------------------- */

static double sqdist(const double* a, const double* b, int d) {
    double s = 0.0;
    for (int j = 0; j < d; ++j) {
        double t = a[j] - b[j];
        s += t * t;
    }
    return s;
}

/* Assignment: each point goes to its nearest centroid (lowest index on a
 * tie).  Centroids are the stored (rounded) ones, mu_s[C][d].  Optional
 * per-point weights w (NULL = 1) only scale the returned objective. */
double orc_assign(const double* x, int32_t n, int32_t d, const double* mu_s, int32_t C,
                  const double* w, int32_t* assign, double* best_dist) {
    double J = 0.0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t best = -1;
        double bd = 0.0;
        for (int32_t c = 0; c < C; ++c) {
            double dist = sqdist(x + (int64_t)i * d, mu_s + (int64_t)c * d, d);
            if (best < 0 || dist < bd) {
                best = c;
                bd = dist;
            }
        }
        assign[i] = best;
        if (best_dist) best_dist[i] = bd;
        J += (w ? w[i] : 1.0) * bd;
    }
    return J;
}

/* Update: every non-empty cluster moves to the (weighted) mean of its
 * members; the stored copy is that mean rounded to the storage dtype.  An
 * empty cluster keeps its previous centroid (a reading: the pages are
 * silent).  counts[c] receives the member count. */
void orc_update(const double* x, int32_t n, int32_t d, const int32_t* assign, const double* w,
                int32_t C, int storage, double* mu, double* mu_s, int32_t* counts) {
    double* sum = (double*)calloc((size_t)C * d, sizeof(double));
    double* wsum = (double*)calloc((size_t)C, sizeof(double));
    for (int32_t c = 0; c < C; ++c) counts[c] = 0;
    for (int32_t i = 0; i < n; ++i) {
        int32_t c = assign[i];
        double wi = w ? w[i] : 1.0;
        counts[c] += 1;
        wsum[c] += wi;
        for (int32_t j = 0; j < d; ++j) sum[(int64_t)c * d + j] += wi * x[(int64_t)i * d + j];
    }
    for (int32_t c = 0; c < C; ++c) {
        if (counts[c] == 0) continue;
        for (int32_t j = 0; j < d; ++j) {
            double m = sum[(int64_t)c * d + j] / wsum[c];
            mu[(int64_t)c * d + j] = m;
            mu_s[(int64_t)c * d + j] = orc_round_storage(m, storage);
        }
    }
    free(sum);
    free(wsum);
}

/* Full run on one block: init from the given point indices, then `iters`
 * rounds of (assign with the stored centroids, update).  J[t] is the
 * objective of assignment round t, measured with the centroids that round
 * used.  No early stop: the iteration count is fixed. */
void orc_kmeans(const double* x, int32_t n, int32_t d, const double* w, int32_t C, int32_t iters,
                int storage, const int32_t* init_idx, double* mu, double* mu_s, int32_t* assign,
                int32_t* counts, double* J) {
    for (int32_t c = 0; c < C; ++c)
        for (int32_t j = 0; j < d; ++j) {
            double v = x[(int64_t)init_idx[c] * d + j];
            mu[(int64_t)c * d + j] = v;
            mu_s[(int64_t)c * d + j] = orc_round_storage(v, storage);
        }
    for (int32_t t = 0; t < iters; ++t) {
        double Jt = orc_assign(x, n, d, mu_s, C, w, assign, NULL);
        if (J) J[t] = Jt;
        orc_update(x, n, d, assign, w, C, storage, mu, mu_s, counts);
    }
}

/* ------------------------------------------------------------------------- */
/* Clustering one block of a unit's cache and writing the unit's state.      */
/* Blocks: [APP] "blockwise", [ABL] block-size rows.  Clusters per block:     */
/* ceil(L / tokens_per_centroid) ([ABL] centroid-ratio rows; reading).        */
/* ------------------------------------------------------------------------- */

/*
 * K, V   : the unit's cache, rows [N][d] (only rows p .. p+L-1 are read).
 * p, L   : first token and length of the block.
 * c0, C  : first global cluster id and number of clusters of the block.
 * Outputs (unit arrays, indexed by global cluster id / token id):
 *   mu[c][d]   key centroid, unrounded mean;    kbar[c][d] stored key centroid
 *   vbar[c][d] stored value centroid = rounded mean of member values (zero
 *              for an empty cluster; it is never used);
 *   sizes[c], offsets[c .. c+C] (positions into token_ids; offsets[c0] = p),
 *   token_ids[p .. p+L-1] member token ids sorted by (cluster, token),
 *   assign[p .. p+L-1] global cluster id of each token, J[iters].
 */
int orc_cluster_block(const double* K, const double* V, int32_t d, int32_t p, int32_t L,
                      int32_t c0, int32_t C, int32_t iters, int storage, uint64_t s0,
                      double* mu, double* kbar, double* vbar, int32_t* sizes, int32_t* offsets,
                      int32_t* token_ids, int32_t* assign, double* J) {
    int32_t* init_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    int32_t* local = (int32_t*)malloc(sizeof(int32_t) * (size_t)L);
    if (!init_idx || !local || orc_init_indices(s0, L, C, init_idx) != 0) {
        free(init_idx);
        free(local);
        return -1;
    }
    const double* Kb = K + (int64_t)p * d;
    orc_kmeans(Kb, L, d, NULL, C, iters, storage, init_idx, mu + (int64_t)c0 * d,
               kbar + (int64_t)c0 * d, local, sizes + c0, J);
    /* value centroids ([APP] "value centroids"): mean of member values */
    for (int32_t c = 0; c < C; ++c) {
        double* vb = vbar + (int64_t)(c0 + c) * d;
        int32_t nc = sizes[c0 + c];
        for (int32_t j = 0; j < d; ++j) vb[j] = 0.0;
        if (nc == 0) continue;
        for (int32_t i = 0; i < L; ++i)
            if (local[i] == c)
                for (int32_t j = 0; j < d; ++j) vb[j] += V[(int64_t)(p + i) * d + j];
        for (int32_t j = 0; j < d; ++j) vb[j] = orc_round_storage(vb[j] / nc, storage);
    }
    /* membership lists, ordered by (cluster, token) */
    int32_t pos = p;
    for (int32_t c = 0; c < C; ++c) {
        offsets[c0 + c] = pos;
        for (int32_t i = 0; i < L; ++i)
            if (local[i] == c) token_ids[pos++] = p + i;
    }
    offsets[c0 + C] = pos;
    for (int32_t i = 0; i < L; ++i) assign[p + i] = c0 + local[i];
    free(init_idx);
    free(local);
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Coarse level of the hierarchy ([APP] "hierarchical variant").  Reading:    */
/* the coarse clusters of a block come from a size-weighted k-means over the  */
/* block's non-empty fine key centroids (weight = fine cluster size), so each */
/* fine cluster sits in exactly one coarse cluster.  Coarse key centroid =    */
/* stored weighted mean of member fine key centroids; coarse value centroid = */
/* stored size-weighted mean of member fine value centroids; coarse size =    */
/* total member tokens.                                                       */
/* ------------------------------------------------------------------------- */

/*
 * fine arrays are the unit's (global ids); the block's fine clusters are
 * [c0, c0+C), its coarse clusters [g0, g0+D).
 * Outputs: cmu[g][d] (unrounded), ckbar[g][d], cvbar[g][d], csizes[g],
 *   parent[c] (global coarse id of fine cluster c, -1 for an empty one),
 *   coffsets[g .. g+D] and cmembers[...] (non-empty fine ids ordered by
 *   (coarse, fine), positions counted from cpos0), J[iters].
 * Returns the number of members written, or < 0 on error.
 */
int orc_coarse_block(const double* kbar, const double* vbar, const int32_t* sizes, int32_t d,
                     int32_t c0, int32_t C, int32_t g0, int32_t D, int32_t iters, int storage,
                     uint64_t s0, int32_t cpos0, double* cmu, double* ckbar, double* cvbar,
                     int32_t* csizes, int32_t* parent, int32_t* coffsets, int32_t* cmembers,
                     double* J) {
    int32_t m = 0;
    for (int32_t c = 0; c < C; ++c) m += sizes[c0 + c] > 0;
    /* Reading: with fewer non-empty fine clusters than coarse ones, only m
     * coarse clusters are seeded; the others stay empty (zero centroids). */
    const int32_t Dfull = D;
    if (D > m) D = m;
    for (int32_t g = D; g < Dfull; ++g) {
        for (int32_t j = 0; j < d; ++j) {
            cmu[(int64_t)(g0 + g) * d + j] = 0.0;
            ckbar[(int64_t)(g0 + g) * d + j] = 0.0;
            cvbar[(int64_t)(g0 + g) * d + j] = 0.0;
        }
        csizes[g0 + g] = 0;
    }
    if (m == 0) {
        for (int32_t c = 0; c < C; ++c) parent[c0 + c] = -1;
        for (int32_t g = 0; g <= Dfull; ++g) coffsets[g0 + g] = cpos0;
        return 0;
    }
    double* pts = (double*)malloc(sizeof(double) * (size_t)m * d);
    double* w = (double*)malloc(sizeof(double) * (size_t)m);
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)m);
    int32_t* init_idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)D);
    int32_t* local = (int32_t*)malloc(sizeof(int32_t) * (size_t)m);
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)D);
    if (!pts || !w || !ids || !init_idx || !local || !counts) {
        free(pts); free(w); free(ids); free(init_idx); free(local); free(counts);
        return -2;
    }
    int32_t k = 0;
    for (int32_t c = 0; c < C; ++c) {
        if (sizes[c0 + c] == 0) continue;
        memcpy(pts + (int64_t)k * d, kbar + (int64_t)(c0 + c) * d, sizeof(double) * d);
        w[k] = (double)sizes[c0 + c];
        ids[k] = c0 + c;
        ++k;
    }
    if (orc_init_indices(s0, m, D, init_idx) != 0) {
        free(pts); free(w); free(ids); free(init_idx); free(local); free(counts);
        return -1;
    }
    orc_kmeans(pts, m, d, w, D, iters, storage, init_idx, cmu + (int64_t)g0 * d,
               ckbar + (int64_t)g0 * d, local, counts, J);
    for (int32_t c = 0; c < C; ++c) parent[c0 + c] = -1;
    for (int32_t i = 0; i < m; ++i) parent[ids[i]] = g0 + local[i];
    int32_t pos = cpos0;
    for (int32_t g = 0; g < D; ++g) {
        double tot = 0.0;
        double* cv = cvbar + (int64_t)(g0 + g) * d;
        for (int32_t j = 0; j < d; ++j) cv[j] = 0.0;
        coffsets[g0 + g] = pos;
        for (int32_t i = 0; i < m; ++i) {
            if (local[i] != g) continue;
            cmembers[pos++] = ids[i];
            tot += w[i];
            for (int32_t j = 0; j < d; ++j) cv[j] += w[i] * vbar[(int64_t)ids[i] * d + j];
        }
        csizes[g0 + g] = (int32_t)tot;
        for (int32_t j = 0; j < d; ++j) cv[j] = tot > 0 ? orc_round_storage(cv[j] / tot, storage) : 0.0;
    }
    for (int32_t g = D; g <= Dfull; ++g) coffsets[g0 + g] = pos;
    free(pts); free(w); free(ids); free(init_idx); free(local); free(counts);
    return pos - cpos0;
}

/* ------------------------------------------------------------------------- */
/* Decode step for one unit (one sequence, one KV head, G query heads).      */
/* ------------------------------------------------------------------------- */

typedef struct {
    double key;
    int32_t id;
} orc_rank_item;

/* Order: larger key first; equal keys by smaller id. */
static int rank_cmp(const void* a, const void* b) {
    const orc_rank_item* x = (const orc_rank_item*)a;
    const orc_rank_item* y = (const orc_rank_item*)b;
    if (x->key > y->key) return -1;
    if (x->key < y->key) return 1;
    return (x->id > y->id) - (x->id < y->id);
}

/* Budgeted selection ([SUM] top-scoring clusters; [HOM] compare the query
 * with the centroids).  Items with size 0 never take part.  Reading: items
 * are taken in order while the running token count stays within the budget;
 * the first item that would overflow it ends the selection.  sel[i] = 1 for
 * selected items.  Returns the number of tokens selected. */
int64_t orc_select(const double* key, const int32_t* size, int32_t n, int64_t budget, int32_t* sel) {
    orc_rank_item* it = (orc_rank_item*)malloc(sizeof(orc_rank_item) * (size_t)(n > 0 ? n : 1));
    int32_t m = 0;
    for (int32_t i = 0; i < n; ++i) {
        sel[i] = 0;
        if (size[i] > 0) {
            it[m].key = key[i];
            it[m].id = i;
            ++m;
        }
    }
    qsort(it, (size_t)m, sizeof(orc_rank_item), rank_cmp);
    int64_t total = 0;
    for (int32_t k = 0; k < m; ++k) {
        int64_t nk = size[it[k].id];
        if (total + nk > budget) break;
        total += nk;
        sel[it[k].id] = 1;
    }
    free(it);
    return total;
}

/* Centroid scores for G query heads: s[g][c] = q_g . kbar_c / sqrt(d), and
 * the group ranking key r[c] = mean over g of s[g][c] (reading: one shared
 * selection per KV head, ranked by the group-mean score). */
void orc_scores(const double* q, int32_t G, int32_t d, const double* kbar, int32_t C, double* s,
                double* r) {
    double scale = 1.0 / sqrt((double)d);
    for (int32_t c = 0; c < C; ++c) {
        double acc_r = 0.0;
        for (int32_t g = 0; g < G; ++g) {
            double dot = 0.0;
            for (int32_t j = 0; j < d; ++j) dot += q[(int64_t)g * d + j] * kbar[(int64_t)c * d + j];
            s[(int64_t)g * C + c] = dot * scale;
            acc_r += s[(int64_t)g * C + c];
        }
        r[c] = acc_r / G;
    }
}

/*
 * Combine ([APP], [SUM], [ABS]): for one query head, with exact logits
 * l_i = q.k_i/sqrt(d) over the exact token set E and the approximate terms of
 * the pseudo set P (cluster size n_c, score s_c, value centroid vbar_c):
 *
 *   out = ( sum_E exp(l_i) v_i + sum_P n_c exp(s_c) vbar_c )
 *       / ( sum_E exp(l_i)     + sum_P n_c exp(s_c) )
 *
 * evaluated with the common factor exp(-M), M the largest exponent, divided
 * out of both sums.  exact[i] = 1 marks E, pseudo[c] = 1 marks P.
 */
void orc_combine(const double* q, int32_t d, const double* K, const double* V, int32_t N,
                 const int32_t* exact, const double* s, const double* vbar, const int32_t* sizes,
                 const int32_t* pseudo, int32_t C, double* out) {
    double scale = 1.0 / sqrt((double)d);
    double* l = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    double M = -INFINITY;
    for (int32_t i = 0; i < N; ++i) {
        if (!exact[i]) continue;
        double dot = 0.0;
        for (int32_t j = 0; j < d; ++j) dot += q[j] * K[(int64_t)i * d + j];
        l[i] = dot * scale;
        if (l[i] > M) M = l[i];
    }
    for (int32_t c = 0; c < C; ++c)
        if (pseudo[c] && s[c] + log((double)sizes[c]) > M) M = s[c] + log((double)sizes[c]);
    double den = 0.0;
    for (int32_t j = 0; j < d; ++j) out[j] = 0.0;
    for (int32_t i = 0; i < N; ++i) {
        if (!exact[i]) continue;
        double e = exp(l[i] - M);
        den += e;
        for (int32_t j = 0; j < d; ++j) out[j] += e * V[(int64_t)i * d + j];
    }
    for (int32_t c = 0; c < C; ++c) {
        if (!pseudo[c]) continue;
        double e = (double)sizes[c] * exp(s[c] - M);
        den += e;
        for (int32_t j = 0; j < d; ++j) out[j] += e * vbar[(int64_t)c * d + j];
    }
    for (int32_t j = 0; j < d; ++j) out[j] = den > 0.0 ? out[j] / den : 0.0;
    free(l);
}

/*
 * One decode step of the flat method for one unit.
 *   q[G][d]; K, V [n_total][d]; clustered tokens are [0, n_clustered), the
 *   tail [n_clustered, n_total) is attended exactly (reading of the online
 *   update: tokens not yet clustered have no centroid to stand in for them).
 *   kbar, vbar [C][d], sizes[C], assign[n_clustered] (global cluster ids).
 *   mode 0: multipole (unselected clusters approximated);
 *   mode 1: unselected clusters omitted (the ablation the pages compare to).
 * Outputs: out[G][d], sel[C] (1 = exact), s[G][C], r[C]; returns tokens
 * selected.
 */
int64_t orc_decode(const double* q, int32_t G, int32_t d, const double* K, const double* V,
                   int32_t n_total, int32_t n_clustered, const double* kbar, const double* vbar,
                   const int32_t* sizes, const int32_t* assign, int32_t C, int64_t budget, int mode,
                   double* out, int32_t* sel, double* s, double* r) {
    orc_scores(q, G, d, kbar, C, s, r);
    int64_t taken = orc_select(r, sizes, C, budget, sel);
    int32_t* exact = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_total > 0 ? n_total : 1));
    int32_t* pseudo = (int32_t*)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    for (int32_t i = 0; i < n_total; ++i) exact[i] = i >= n_clustered ? 1 : sel[assign[i]];
    for (int32_t c = 0; c < C; ++c) pseudo[c] = (mode == 0) && sizes[c] > 0 && !sel[c];
    for (int32_t g = 0; g < G; ++g)
        orc_combine(q + (int64_t)g * d, d, K, V, n_total, exact, s + (int64_t)g * C, vbar, sizes,
                    pseudo, C, out + (int64_t)g * d);
    free(exact);
    free(pseudo);
    return taken;
}

/*
 * One decode step of the two-level method for one unit.
 *   Coarse scores pick candidate coarse clusters (budget cand_budget tokens);
 *   fine clusters inside the candidates are scored and selected under
 *   `budget`; the exact set is the selected fine clusters' tokens plus the
 *   tail; the approximate set is every unselected non-empty fine cluster
 *   inside a candidate plus every non-candidate non-empty coarse cluster.
 * forced_csel / forced_sel (may be NULL) replace the candidate and fine
 * selections (to evaluate the combine for a given selection).
 * Outputs: out[G][d], csel[D] (candidates), sel[C] (selected fine), s[G][C]
 *   (fine scores; only candidates' entries are computed, others zero),
 *   cs[G][D], r_out[C] (may be NULL); returns tokens selected.
 */
int64_t orc_decode_hier(const double* q, int32_t G, int32_t d, const double* K, const double* V,
                        int32_t n_total, int32_t n_clustered, const double* kbar,
                        const double* vbar, const int32_t* sizes, const int32_t* assign,
                        const int32_t* parent, int32_t C, const double* ckbar,
                        const double* cvbar, const int32_t* csizes, int32_t D,
                        int64_t cand_budget, int64_t budget, const int32_t* forced_csel,
                        const int32_t* forced_sel, double* out, int32_t* csel, int32_t* sel, double* s,
                        double* cs, double* r_out) {
    double* cr = (double*)malloc(sizeof(double) * (size_t)(D > 0 ? D : 1));
    orc_scores(q, G, d, ckbar, D, cs, cr);
    if (forced_csel)
        for (int32_t k = 0; k < D; ++k) csel[k] = forced_csel[k];
    else
        orc_select(cr, csizes, D, cand_budget, csel);
    /* fine scores for candidate members only */
    double* r = (double*)malloc(sizeof(double) * (size_t)(C > 0 ? C : 1));
    int32_t* csize_f = (int32_t*)malloc(sizeof(int32_t) * (size_t)(C > 0 ? C : 1));
    double scale = 1.0 / sqrt((double)d);
    for (int32_t c = 0; c < C; ++c) {
        int in_cand = sizes[c] > 0 && parent[c] >= 0 && csel[parent[c]];
        csize_f[c] = in_cand ? sizes[c] : 0;
        r[c] = 0.0;
        for (int32_t g = 0; g < G; ++g) {
            double v = 0.0;
            if (in_cand) {
                double dot = 0.0;
                for (int32_t j = 0; j < d; ++j) dot += q[(int64_t)g * d + j] * kbar[(int64_t)c * d + j];
                v = dot * scale;
            }
            s[(int64_t)g * C + c] = v;
            r[c] += v;
        }
        r[c] /= G;
    }
    int64_t taken = 0;
    if (forced_sel) {
        for (int32_t c = 0; c < C; ++c) {
            sel[c] = forced_sel[c];
            if (sel[c]) taken += sizes[c];
        }
    } else {
        taken = orc_select(r, csize_f, C, budget, sel);
    }
    if (r_out)
        for (int32_t c = 0; c < C; ++c) r_out[c] = r[c];
    int32_t* exact = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n_total > 0 ? n_total : 1));
    for (int32_t i = 0; i < n_total; ++i) exact[i] = i >= n_clustered ? 1 : sel[assign[i]];
    /* Approximate items: fine (inside candidates, unselected) then coarse
     * (not candidates), combined through one call by concatenation. */
    int32_t P = C + D;
    double* ps = (double*)malloc(sizeof(double) * (size_t)P);
    double* pv = (double*)malloc(sizeof(double) * (size_t)P * d);
    int32_t* pn = (int32_t*)malloc(sizeof(int32_t) * (size_t)P);
    int32_t* pm = (int32_t*)malloc(sizeof(int32_t) * (size_t)P);
    for (int32_t g = 0; g < G; ++g) {
        for (int32_t c = 0; c < C; ++c) {
            ps[c] = s[(int64_t)g * C + c];
            pn[c] = sizes[c];
            pm[c] = csize_f[c] > 0 && !sel[c];
            memcpy(pv + (int64_t)c * d, vbar + (int64_t)c * d, sizeof(double) * d);
        }
        for (int32_t k = 0; k < D; ++k) {
            ps[C + k] = cs[(int64_t)g * D + k];
            pn[C + k] = csizes[k];
            pm[C + k] = csizes[k] > 0 && !csel[k];
            memcpy(pv + (int64_t)(C + k) * d, cvbar + (int64_t)k * d, sizeof(double) * d);
        }
        orc_combine(q + (int64_t)g * d, d, K, V, n_total, exact, ps, pv, pn, pm, P,
                    out + (int64_t)g * d);
    }
    free(cr); free(r); free(csize_f); free(exact); free(ps); free(pv); free(pn); free(pm);
    return taken;
}

/* Dense softmax attention of one query over N keys: the textbook definition,
 * out = sum_i softmax_i(q.k_i/sqrt(d)) v_i.  Used as an independent check. */
void orc_dense(const double* q, int32_t d, const double* K, const double* V, int32_t N, double* out) {
    double scale = 1.0 / sqrt((double)d);
    double M = -INFINITY;
    double* l = (double*)malloc(sizeof(double) * (size_t)(N > 0 ? N : 1));
    for (int32_t i = 0; i < N; ++i) {
        double dot = 0.0;
        for (int32_t j = 0; j < d; ++j) dot += q[j] * K[(int64_t)i * d + j];
        l[i] = dot * scale;
        if (l[i] > M) M = l[i];
    }
    double den = 0.0;
    for (int32_t j = 0; j < d; ++j) out[j] = 0.0;
    for (int32_t i = 0; i < N; ++i) {
        double e = exp(l[i] - M);
        den += e;
        for (int32_t j = 0; j < d; ++j) out[j] += e * V[(int64_t)i * d + j];
    }
    for (int32_t j = 0; j < d; ++j) out[j] = N > 0 ? out[j] / den : 0.0;
    free(l);
}
