// decode.hip -- one Multipole Attention decode step on gfx950.
//
// Pages: mlsanity.com paper page, "Abstract (arXiv)" (centroids identify the
// important keys and approximate the rest); atlas.scime.ai summary, opening
// sentence (exact attention on the top-scoring clusters, centroid attention
// for the rest) and "Approach" (unselected clusters contribute through their
// value centroids).  The approximate term of an unselected cluster c is
// n_c * exp(q . Kbar_c / sqrt(d)) on Vbar_c, in numerator and denominator.
//
// Launches:
//   score   -- s[c][g] = q_g . Kbar_c / sqrt(d) for every item, and one
//              16-byte record per item for the cut: group-mean ranking key,
//              budget weight (size), first member position, member rows;
//   select  -- one workgroup per unit takes the budget cut (longest prefix of
//              the (key desc, id asc) order whose weights fit the budget) with
//              a radix select, and writes the selected clusters (id, first
//              member position, prefix of member rows) and a bitmask of them;
//              the SAME launch carries the approximate term: further
//              workgroups stream Vbar and add the term of EVERY non-empty
//              cluster (logit s + ln n, value Vbar) into one partial softmax
//              state per chunk of 256 clusters, so the cut's latency hides
//              behind that stream;
//   attend  -- split-K online softmax over the exact rows of the selected
//              clusters (gathered K/V) and the unclustered tail, minus the
//              approximate terms of the selected clusters;
//   merge   -- log-sum-exp merge of the attend splits and the chunk partials.
// All softmax states are kept in base-2 exponent units with fp32 sums.
//
// Adding every cluster's approximate term and removing the selected ones
// afterwards makes the approximate term a dense, selection-independent
// stream.  The cancellation is harmless: by convexity of exp, a cluster's
// approximate term never exceeds the sum of its members' exact terms (up to
// the storage rounding of the centroids), so the removed mass is at most the
// exact mass that replaces it and the rounding error of the difference stays
// within a few fp32 units of the final denominator.  The removed term is
// recomputed from the same stored score and size, so it matches the added one
// to the last rounding of exp2.
//
// Kernel boundaries carry the cross-workgroup dependencies: a device-scope
// fence per workgroup (write back + invalidate of an XCD's L2) serialises and
// costs far more than a launch on this chip.
#include <math.h>

#include "attn.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

// Combines the 16 row groups of a 256-thread workgroup (4 per wave through
// lane shuffles, then the 4 waves through LDS, in wave order) and writes the
// workgroup's partial to slot `slot`.  Every thread of the workgroup calls it.
template <int G>
__device__ __forceinline__ void finish_partial(SoftState<G>& st, float (*s_red)[G][kHeadDim + 2], float* part_ml,
                                               float* part_acc, int unit, int slot, int P) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
#pragma unroll
    for (int step = 16; step <= 32; step <<= 1) {
        float om[G], ol[G], oacc[G][8];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            om[g] = shfl_xor_f(st.m[g], step);
            ol[g] = shfl_xor_f(st.l[g], step);
#pragma unroll
            for (int e = 0; e < 8; ++e) oacc[g][e] = shfl_xor_f(st.acc[g][e], step);
        }
        merge_state<G>(st, om, ol, oacc);
    }
    __syncthreads();
    if (rg == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
#pragma unroll
            for (int e = 0; e < 8; ++e) s_red[wave][g][li * 8 + e] = st.acc[g][e];
            if (li == 0) {
                s_red[wave][g][kHeadDim] = st.m[g];
                s_red[wave][g][kHeadDim + 1] = st.l[g];
            }
        }
    }
    __syncthreads();
    for (int e = tid; e < G * kHeadDim; e += 256) {
        const int g = e / kHeadDim, dd = e % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < 4; ++w) M = fmaxf(M, s_red[w][g][kHeadDim]);
        float l = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const float wt = __builtin_amdgcn_exp2f(s_red[w][g][kHeadDim] - M);
                l = fmaf(s_red[w][g][kHeadDim + 1], wt, l);
                acc = fmaf(s_red[w][g][dd], wt, acc);
            }
        }
        const size_t pidx = part_index(unit, G, g, P, slot);
        part_acc[pidx * kHeadDim + dd] = acc;
        if (dd == 0) {
            part_ml[pidx * 2] = M;
            part_ml[pidx * 2 + 1] = l;
        }
    }
}

// ---------------------------------------------------------------------------
// score: workgroup (chunk, unit) scores 256 items, 16 lanes per centroid row,
// 16 rows per lane group in flight (8 in fp32, two passes); row group (wave,
// rg) takes items 16 u + 4 wave + rg, so the waves read one interleaved
// stream (separate per-wave streams cost HBM efficiency).  Items are
// cluster ids, or the member rows of a previous selection (the fine clusters
// inside the coarse candidates of the two-level method).  Thread t writes the
// cut record of item t of the chunk (its fields load at the start; the key
// comes through LDS).
// ---------------------------------------------------------------------------
constexpr int kScoreChunk = 256;  // items per workgroup
constexpr int kListCap = 1024;    // selection-list entries staged in LDS

template <typename T, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    __shared__ int32_t s_pre[kListCap + 1];
    __shared__ int32_t s_off[kListCap];
    __shared__ float s_key[kScoreChunk];
    const int unit = blockIdx.y;
    int n = a.n_items;
    if (a.n_items_dev) n = min(n, a.n_items_dev[unit * 4]);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int c0 = blockIdx.x * kScoreChunk;
    const int i0 = c0 + wave * 4;  // the waves interleave by 4 items: one stream per workgroup
    if (c0 >= n) return;  // uniform across the workgroup

    // items through a selection list: stage its member-row prefix
    const int32_t* mem = a.members ? a.members + (size_t)unit * a.cent_rows : nullptr;
    const int32_t* lpre = nullptr;
    const int32_t* loff = nullptr;
    int nl = 0;
    if (a.list_pre) {
        nl = a.list_counts[unit * 4 + 1];
        const int32_t* gpre = a.list_pre + (size_t)unit * (a.list_stride + 1);
        const int32_t* goff = a.list_off + (size_t)unit * a.list_stride;
        if (nl <= kListCap) {
            for (int k = tid; k <= nl; k += 256) {
                s_pre[k] = gpre[k];
                if (k < nl) s_off[k] = goff[k];
            }
            __syncthreads();
            lpre = s_pre;
            loff = s_off;
        } else {
            lpre = gpre;
            loff = goff;
        }
    }
    auto item_id = [&](int i) -> int {
        if (!lpre) return i;
        const int k = upper_index(lpre, nl, i);
        return mem[loff[k] + i - lpre[k]];
    };
    // record fields of item c0 + tid, loaded up front
    const int my_item = c0 + tid;
    int my_id = 0, my_sz = 0, my_o0 = 0, my_o1 = 0;
    if (my_item < n) {
        my_id = item_id(my_item);
        const int32_t* ofu = a.offsets + (size_t)unit * a.off_stride;
        my_sz = a.sizes[(size_t)unit * a.cent_rows + my_id];
        my_o0 = ofu[my_id];
        my_o1 = ofu[my_id + 1];
    }

    if constexpr (sizeof(T) == 2) {
        // bf16: 16 items per matrix-core product; group u of wave w holds
        // items c0 + 64 u + 16 w .. + 16 (lane l loads item l % 16 of them)
        const int b = unit / a.Hkv, h = unit % a.Hkv;
        const bf16_t* qg = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim;
        QOperand qop;
        load_qop<G>(qop, qg, lane);
        const bf16_t* cu = reinterpret_cast<const bf16_t*>(a.cent) + (size_t)unit * a.cent_rows * kHeadDim;
        int cid[4];
        Slice8<bf16_t> rows[4][4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = c0 + u * 64 + wave * 16 + li;
            cid[u] = item_id(i < n ? i : c0);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) load_row_blocks(rows[u], cu + (size_t)cid[u] * kHeadDim, lane);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const f32x4v d = mfma_scores(rows[u], qop);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int r = 4 * rg + e;  // item of the 16 whose scores lane (rg, li) holds
                const int i = c0 + u * 64 + wave * 16 + r;
                const int id = __shfl(cid[u], r, kWave);
                const float sv = d[e] * kInvSqrtD;
                const float key = head_mean<G>(sv);
                if (i < n) {
                    if (li < G) a.s_out[((size_t)unit * a.cent_rows + id) * G + li] = sv;
                    if (li == 0) s_key[i - c0] = key;
                }
            }
        }
    } else if (i0 < n) {
        const int b = unit / a.Hkv, h = unit % a.Hkv;
        QSlice<T> qv[G];
        const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g].load(qb + (size_t)g * kHeadDim);
        const T* cu = reinterpret_cast<const T*>(a.cent) + (size_t)unit * a.cent_rows * kHeadDim + li * 8;
        constexpr int R = sizeof(T) == 2 ? 16 : 8;
#pragma unroll 1
        for (int pass = 0; pass < 16 / R; ++pass) {
            const int ib = i0 + pass * 16 * R;
            if (ib >= n) break;  // uniform across the wave
            int cid[R];
            Slice8<T> row[R];
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int i = ib + u * 16 + rg;
                cid[u] = item_id(i < n ? i : ib);
            }
#pragma unroll
            for (int u = 0; u < R; ++u) row[u].load(cu + (size_t)cid[u] * kHeadDim);
#pragma unroll
            for (int u = 0; u < R; ++u) {
                const int i = ib + u * 16 + rg;
                float sg[G];
                float r = 0.f;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    sg[g] = row16_sum(dot8(qv[g], row[u])) * kInvSqrtD;
                    r += sg[g];
                }
                r *= 1.0f / G;
                if (i < n) {
                    float* so = a.s_out + ((size_t)unit * a.cent_rows + cid[u]) * G;
                    float mine = sg[0];
#pragma unroll
                    for (int g = 1; g < G; ++g) mine = li == g ? sg[g] : mine;
                    if (li < G) so[li] = mine;
                    if (li == 0) s_key[i - c0] = r;
                }
            }
        }
    }
    __syncthreads();
    if (my_item < n) {
        const size_t o = (size_t)unit * a.rs_stride + my_item;
        a.rs_out[o] = make_int4(__float_as_int(s_key[tid]), my_sz, my_o0, my_o1 - my_o0);
        if (a.ids_out) a.ids_out[o] = my_id;
    }
}

// ---------------------------------------------------------------------------
// select: budget cut of one unit by one 256-thread workgroup.  Thread t owns
// items 8 t .. 8 t + 7 of each tile of 2048 (record in registers).  Four
// 8-bit radix passes over the order-preserving key bits find the cut value:
// pass p adds the weights of the items still matching the prefix into its own
// LDS histogram (all four are cleared up front, so a pass needs one barrier),
// then every wave scans that histogram from the top digit down to the budget
// left, and all reach the same digit.  Items above the cut value are
// selected; items equal to it are taken in item order while they fit.  One
// workgroup scan places the selected items in item order.
// ---------------------------------------------------------------------------
constexpr int kSelItems = 8;                 // items per thread per tile
constexpr int kSelTileN = 256 * kSelItems;   // items per tile
constexpr int kMaskWords = 1024;             // LDS bitmask capacity (32768 ids)

struct SelItems {
    uint32_t key[kSelItems];
    int32_t sz[kSelItems], off[kSelItems], rows[kSelItems];
};

__device__ __forceinline__ void load_items(const SelectArgs& a, int unit, int n, int base, SelItems& it) {
    const int4* rs = a.rs + (size_t)unit * a.rs_stride;
    const int t0 = base + threadIdx.x * kSelItems;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        const int4 v = t0 + j < n ? rs[t0 + j] : make_int4(0, 0, 0, 0);
        it.key[j] = order_key(__int_as_float(v.x));
        it.sz[j] = v.y;
        it.off[j] = v.z;
        it.rows[j] = v.w;
    }
}

__device__ __forceinline__ void select_unit(const SelectArgs& a, int unit) {
    __shared__ int hist[4][256];
    __shared__ int scan_lds[16];
    __shared__ uint32_t s_mask[kMaskWords];
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    int n = a.n_items;
    if (a.n_items_dev) n = min(n, a.n_items_dev[unit * 4]);
    const int mwords = (a.mask_bits + 31) >> 5;

    SelItems it;
    const bool resident = n <= kSelTileN;
    if (resident) load_items(a, unit, n, 0, it);
#pragma unroll
    for (int p = 0; p < 4; ++p) hist[p][tid] = 0;
    for (int w = tid; w < mwords; w += 256) s_mask[w] = 0;
    __syncthreads();

    uint32_t prefix = 0, mask = 0;
    int R = a.budget;
    bool done = false;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
        for (int base = 0; base < n; base += kSelTileN) {
            if (!resident) load_items(a, unit, n, base, it);
#pragma unroll
            for (int j = 0; j < kSelItems; ++j)
                if (it.sz[j] > 0 && (it.key[j] & mask) == prefix)
                    atomicAdd(&hist[p][(it.key[j] >> shift) & 255u], it.sz[j]);
        }
        __syncthreads();
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = hist[p][255 - (4 * lane + j)];
        int total;
        int run = wave_exclusive_sum(v[0] + v[1] + v[2] + v[3], total);
        if (total <= R) {  // the same in every wave
            done = true;
            break;
        }
        int found = -1, cum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (found < 0 && run <= R && R < run + v[j]) {
                found = 255 - (4 * lane + j);
                cum = run;
            }
            run += v[j];
        }
        const uint64_t bal = __ballot(found >= 0);
        const int src = __ffsll((long long)bal) - 1;
        const int digit = lane_value(found, src);
        R -= lane_value(cum, src);
        prefix |= (uint32_t)digit << shift;
        mask |= 0xFFu << shift;
    }
    const uint32_t tau = prefix;

    const int32_t* gids = a.ids ? a.ids + (size_t)unit * a.rs_stride : nullptr;
    int32_t* sid = a.sel_ids + (size_t)unit * a.sel_stride;
    int32_t* soff = a.sel_off + (size_t)unit * a.sel_stride;
    int32_t* spre = a.sel_rowpre + (size_t)unit * (a.sel_stride + 1);
    int32_t* dbg = a.dbg_selected ? a.dbg_selected + (size_t)unit * a.dbg_stride : nullptr;
    int carry_rows = 0, carry_sel = 0, carry_tie = 0;
    // With an id list (the candidates' fine clusters, listed by coarse id)
    // the item order is not the id order: when several items carry the cut
    // value, each of them sums the tied sizes of lower ids over all items
    // (ties are rare).  The count of tied items comes first.
    bool by_id = false;
    if (!done && gids) {
        int tied = 0;
        for (int base = 0; base < n; base += kSelTileN) {
            if (!resident) load_items(a, unit, n, base, it);
            int h = 0;
#pragma unroll
            for (int j = 0; j < kSelItems; ++j) h += it.sz[j] > 0 && it.key[j] == tau;
            int4 tt;
            block256_exclusive_sum4(make_int4(h, 0, 0, 0), tt, scan_lds);
            tied += tt.x;
        }
        by_id = tied > 1;
    }
    const int4* rsu = a.rs + (size_t)unit * a.rs_stride;
    for (int base = 0; base < n; base += kSelTileN) {
        if (!resident) load_items(a, unit, n, base, it);
        const int t0 = base + tid * kSelItems;
        int tie_local = 0;
        if (!done) {
#pragma unroll
            for (int j = 0; j < kSelItems; ++j)
                if (it.sz[j] > 0 && it.key[j] == tau) tie_local += it.sz[j];
        }
        int run_tie = carry_tie;
        if (!done && !by_id) {
            // usually a single item carries the cut value: then no scan is needed
            const int holders = __syncthreads_count(tie_local > 0);
            if (holders > 1 || !resident) {
                int4 tt;
                run_tie += block256_exclusive_sum4(make_int4(tie_local, 0, 0, 0), tt, scan_lds).x;
                carry_tie += tt.x;
            }
        }
        uint32_t selbits = 0;
        int s_local = 0, rows_local = 0;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            const int sz = it.sz[j];
            const uint32_t u = it.key[j];
            bool sel;
            if (done) {
                sel = u >= prefix;
            } else {
                const bool tie = u == tau && sz > 0;
                int before = run_tie;
                if (tie && by_id) {
                    before = 0;
                    const int me = gids[t0 + j];
                    for (int i = 0; i < n; ++i) {
                        const int4 v = rsu[i];
                        if (v.y > 0 && order_key(__int_as_float(v.x)) == tau && gids[i] < me) before += v.y;
                    }
                }
                sel = u > tau || (tie && before + sz <= R);
                if (tie) run_tie += sz;
            }
            sel = sel && sz > 0;
            selbits |= (uint32_t)sel << j;
            s_local += sel;
            rows_local += sel ? it.rows[j] : 0;
        }
        int id[kSelItems];
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) id[j] = t0 + j < n ? (gids ? gids[t0 + j] : t0 + j) : 0;
        int4 tot;
        const int4 ex = block256_exclusive_sum4(make_int4(s_local, rows_local, 0, 0), tot, scan_lds);
        int k = carry_sel + ex.x, ro = carry_rows + ex.y;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            if ((selbits >> j) & 1u) {
                sid[k] = id[j];
                soff[k] = it.off[j];
                spre[k] = ro;
                ++k;
                ro += it.rows[j];
                atomicOr(&s_mask[id[j] >> 5], 1u << (id[j] & 31));
            }
            if (dbg && t0 + j < n) dbg[id[j]] = (selbits >> j) & 1u;
        }
        carry_sel += tot.x;
        carry_rows += tot.y;
    }
    __syncthreads();
    uint32_t* gmask = a.selmask + (size_t)unit * a.mask_stride;
    for (int w = tid; w < mwords; w += 256) gmask[w] = s_mask[w];
    if (tid == 0) {
        spre[carry_sel] = carry_rows;
        int32_t* cnt = a.counts + unit * 4;
        cnt[0] = carry_rows;
        cnt[1] = carry_sel;
        cnt[2] = 0;
        cnt[3] = 0;
    }
}

// ---------------------------------------------------------------------------
// Approximate term of every non-empty item of a chunk of 256 items, folded
// into the softmax state of the attend workgroup that owns the chunk.  Thread
// t takes item t's logits lambda_g = s_g log2(e) + log2(n) (base 2) and, after
// a workgroup maximum, its weights 2^(lambda - m) go to LDS (0 for absent or
// empty items); the row groups then add the value centroids they loaded at
// the start of the workgroup.
// ---------------------------------------------------------------------------
template <int G>
struct ChunkMeta {  // item c0 + tid of a chunk
    float s[G];
    int n, c;
};

template <int G>
__device__ __forceinline__ void chunk_meta_issue(ChunkMeta<G>& cm, const PseudoArgs& a, int unit, int chunk, int n) {
    const int c0 = chunk * kScoreChunk, i = c0 + threadIdx.x;
    const int32_t* ids = a.ids ? a.ids + (size_t)unit * a.ids_stride : nullptr;
    // absent items read item c0's row (weight 0)
    cm.c = ids ? ids[i < n ? i : c0] : (i < n ? i : c0);
    cm.n = i < n ? a.sizes[(size_t)unit * a.rows + cm.c] : 0;
    const float* su = a.s + ((size_t)unit * a.rows + cm.c) * G;
#pragma unroll
    for (int g = 0; g < G; ++g) cm.s[g] = su[g];
}

// Weights and ids of the chunk to LDS.  The state's reference first moves to
// max(m, M) (M = the chunk maximum per head; the reference is the same in
// every row group while only chunks have been added), and the weights are
// 2^(lambda - m) relative to it (0 for absent or empty items).  Ends with a
// barrier.
template <int G>
__device__ __forceinline__ void chunk_weights(SoftState<G>& st, const ChunkMeta<G>& cm, float (*s_w)[G],
                                              float (*s_wmax)[G]) {
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    float lg[G];
    const float l2n = log2_count(cm.n > 0 ? cm.n : 1);
#pragma unroll
    for (int g = 0; g < G; ++g) lg[g] = cm.n > 0 ? fmaf(cm.s[g], kLog2e, l2n) : -INFINITY;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float m = lg[g];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, shfl_xor_f(m, o));
        if (lane == 0) s_wmax[wave][g] = m;
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = fmaxf(fmaxf(s_wmax[0][g], s_wmax[1][g]), fmaxf(s_wmax[2][g], s_wmax[3][g]));
        if (M > st.m[g]) {
            const float sc = __builtin_amdgcn_exp2f(st.m[g] - M);
            st.l[g] *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[g][e] *= sc;
            st.m[g] = M;
        }
        s_w[tid][g] = lg[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lg[g] - st.m[g]);
    }
    __syncthreads();
}

__global__ __launch_bounds__(256) void select_kernel(SelectArgs sa) { select_unit(sa, blockIdx.x); }

// ---------------------------------------------------------------------------
// attend: workgroup (split, unit), 4 waves, 16 lanes per row, 8 dims a lane.
// Each row group keeps its own softmax state over the rows it visits, 2 rows
// per step with the next steps' rows already in flight.  Exact rows: split s
// takes rows [E s / S, E (s + 1) / S) of the selected clusters' member rows
// (found by binary search of the row prefix) and its share of the unclustered
// tail; it also removes, for its share of each selected list, the
// approximate terms added for those clusters (the first step's loads go out
// ahead of the exact rows).
// ---------------------------------------------------------------------------
constexpr int kAttCap = 512;   // staged exact rows per pass
constexpr int kAttDepth = 2;   // row steps in flight per wave
constexpr int kSpec = 256;     // selection entries staged before the counts are known

// Removal data of 2 selected clusters per row group: list entries base + 4 u
// + rg (u = 0, 1) of [k0, k1).
template <typename T, int G>
struct SubBuf {
    Slice8<T> v[2];
    float lg[2][G];
};

template <typename T, int G>
__device__ __forceinline__ void load_sub(SubBuf<T, G>& sb, const SubSrc& ss, const int32_t* ids, int unit, int k0,
                                         int k1, int base, int rg, int li) {
    const float* su = ss.s + (size_t)unit * ss.rows * G;
    const int32_t* szu = ss.sizes + (size_t)unit * ss.rows;
    const T* vb = reinterpret_cast<const T*>(ss.vbar) + (size_t)unit * ss.rows * kHeadDim + li * 8;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int k = base + u * 4 + rg;
        const bool ok = k < k1;
        const int c = ids[ok ? k : k0];
        const float l2n = log2_count(szu[c]);  // selected: n >= 1
        sb.v[u].load(vb + (size_t)c * kHeadDim);
#pragma unroll
        for (int g = 0; g < G; ++g) sb.lg[u][g] = ok ? fmaf(su[(size_t)c * G + g], kLog2e, l2n) : -INFINITY;
    }
}

template <int G>
constexpr int attend_lds_bytes() {
    // the chunk weights and their maxima alias the final reduction area
    static_assert(4 * (kHeadDim + 2) >= kScoreChunk + 4, "chunk weights must fit the reduction area");
    return (kAttCap + (kListCap + 1) + 2 * kListCap + 4 * G * (kHeadDim + 2)) * 4;
}

template <typename T, int G>
__device__ __forceinline__ void attend_split(const AttendArgs& a, int split, int unit, char* lds) {
    constexpr int D = kAttDepth;
    int32_t* s_row = reinterpret_cast<int32_t*>(lds);
    int32_t* s_pre = s_row + kAttCap;
    int32_t* s_off = s_pre + kListCap + 1;
    int32_t* s_ids = s_off + kListCap;
    float (*s_red)[G][kHeadDim + 2] = reinterpret_cast<float (*)[G][kHeadDim + 2]>(s_ids + kListCap);
    float (*s_w)[G] = reinterpret_cast<float (*)[G]>(&s_red[0][0][0]);
    float (*s_wmax)[G] = s_w + kScoreChunk;

    const int S = a.S;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    const float qscale = kInvSqrtD * kLog2e;

    // approximate-term chunk of this split: chunk s over the sources (the
    // launcher makes S >= the number of chunks)
    int n_chunks = 0;
    for (int k = 0; k < a.n_pseudo; ++k) n_chunks += a.pseudo[k].chunks;
    auto locate = [&](int cg, int& k, int& ch) {
        k = 0;
        ch = cg;
        while (k + 1 < a.n_pseudo && ch >= a.pseudo[k].chunks) ch -= a.pseudo[k++].chunks;
    };
    auto items_of = [&](const PseudoArgs& ps) {
        return ps.n_items_dev ? min(ps.n_items, ps.n_items_dev[unit * 4]) : ps.n_items;
    };
    int rk = 0, rch = 0, rn = 0;
    bool has_chunk = false;
    ChunkMeta<G> cm;
    Slice8<T> pv[16];  // value centroids of chunk items 16 u + 4 wave + rg
    if (split < n_chunks) {
        locate(split, rk, rch);
        const PseudoArgs& ps = a.pseudo[rk];
        rn = items_of(ps);
        has_chunk = rch * kScoreChunk < rn;
        if (has_chunk) {
            // loads first: they are in flight while the selection is staged
            const int c0 = rch * kScoreChunk;
            const int32_t* pids = ps.ids ? ps.ids + (size_t)unit * ps.ids_stride : nullptr;
            const T* vb = reinterpret_cast<const T*>(ps.vbar) + (size_t)unit * ps.rows * kHeadDim + li * 8;
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                const int i = c0 + u * 16 + wave * 4 + rg;
                const int ii = i < rn ? i : c0;  // absent items read item c0 (weight 0)
                pv[u].load(vb + (size_t)(pids ? pids[ii] : ii) * kHeadDim);
            }
            chunk_meta_issue<G>(cm, ps, unit, rch, rn);
        }
    }

    // selection of the unit: member-row prefix, first member and id of each
    // selected cluster.  The first kSpec entries load beside the counts.
    const int32_t* gpre = a.sel_rowpre + (size_t)unit * (a.sel_stride + 1);
    const int32_t* goff = a.sel_off + (size_t)unit * a.sel_stride;
    const int32_t* gids = a.n_sub > 0 ? a.sa.ids + (size_t)unit * a.sa.ids_stride : nullptr;
    const int spec = min(kSpec, a.sel_stride);
    if (tid < spec) {
        s_off[tid] = goff[tid];
        if (gids) s_ids[tid] = gids[tid];
    }
    if (tid <= spec) s_pre[tid] = gpre[tid];
    if (tid == 0 && spec == kSpec) s_pre[kSpec] = gpre[kSpec];
    const int E = a.counts[unit * 4];
    const int nsel = a.counts[unit * 4 + 1];
    const bool staged = nsel <= kListCap;
    if (staged && nsel > spec) {
        for (int k = spec + 1 + tid; k <= nsel; k += 256) s_pre[k] = gpre[k];
        for (int k = spec + tid; k < nsel; k += 256) {
            s_off[k] = goff[k];
            if (gids) s_ids[k] = gids[k];
        }
    }
    const int32_t* pre = staged ? s_pre : gpre;
    const int32_t* off = staged ? s_off : goff;
    const int32_t* sids = staged ? s_ids : gids;
    const int e0 = (int)((int64_t)E * split / S), e1 = (int)((int64_t)E * (split + 1) / S);
    SoftState<G> st;
    st.init();
    const size_t ubase = (size_t)unit * a.Nmax * kHeadDim + li * 8;
    const T* Kx = reinterpret_cast<const T*>(a.Kx) + ubase;
    const T* Vx = reinterpret_cast<const T*>(a.Vx) + ubase;
    const int32_t* tids = a.token_ids ? a.token_ids + (size_t)unit * a.Nmax : nullptr;
    __syncthreads();

    // ---- the chunk's approximate terms: weights to LDS, then the rows ------
    if (has_chunk) {
        chunk_weights<G>(st, cm, s_w, s_wmax);
#pragma unroll
        for (int u = 0; u < 16; ++u) {
            float x[8];
            pv[u].unpack(x);
            const int r = u * 16 + wave * 4 + rg;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float w = s_w[r][g];
                st.l[g] += w;
#pragma unroll
                for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(w, x[e], st.acc[g][e]);
            }
        }
    }
    // ---- the first batch of exact rows ------------------------------------
    int c0 = e0, cnt = min(kAttCap, e1 - e0);
    if (cnt > 0) stage_exact(s_row, pre, off, nsel, tids, c0, cnt);
    else if (tid == 0) s_row[0] = tids ? tids[0] : 0;  // masked ring steps read a valid row
    __syncthreads();

    const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
    QSlice<T> qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qs[g].load(qb + (size_t)g * kHeadDim);

    // ---- removals of the first list, first step: loads issued first -------
    SubBuf<T, G> sub;
    int sk0 = 0, sk1 = 0;
    if (a.n_sub > 0) {
        sk0 = (int)((int64_t)nsel * split / S);
        sk1 = (int)((int64_t)nsel * (split + 1) / S);
        if (sk0 < sk1) load_sub<T, G>(sub, a.sa, sids, unit, sk0, sk1, sk0 + wave * 8, rg, li);
    }
    const bool sub_pending = a.n_sub > 0 && sk0 < sk1;
    __builtin_amdgcn_sched_barrier(0);

    // ---- exact rows through a ring of D steps in flight.  The loop body has
    //      no branches, so the compiler's wait counts stay exact: steps past
    //      the end load a valid row (staged row 0) and are masked out. ------
    RowBuf<T> ring[D];
#pragma unroll
    for (int j = 0; j < D; ++j) {
        load_rows<T>(ring[j], s_row, cnt, j, wave, rg, Kx, Vx);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (sub_pending) absorb2<T, G, true>(st, sub.lg, sub.v);
    {
        const int steps = (cnt + 31) / 32;
        for (int it = 0; it < steps; it += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                exact_step<T, G>(st, qs, qscale, ring[j]);
                load_rows<T>(ring[j], s_row, cnt, it + j + D, wave, rg, Kx, Vx);
                __builtin_amdgcn_sched_barrier(0);  // keep the ring order: no load sinks
            }
        }
    }
    // ---- further batches of exact rows ------------------------------------
    for (c0 += kAttCap; c0 < e1; c0 += kAttCap) {
        cnt = min(kAttCap, e1 - c0);
        __syncthreads();
        stage_exact(s_row, pre, off, nsel, tids, c0, cnt);
        __syncthreads();
#pragma unroll
        for (int j = 0; j < D; ++j) {
            load_rows<T>(ring[j], s_row, cnt, j, wave, rg, Kx, Vx);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int steps = (cnt + 31) / 32;
        for (int it = 0; it < steps; it += D) {
#pragma unroll
            for (int j = 0; j < D; ++j) {
                exact_step<T, G>(st, qs, qscale, ring[j]);
                load_rows<T>(ring[j], s_row, cnt, it + j + D, wave, rg, Kx, Vx);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
    }
    // ---- unclustered tail, attended exactly ------------------------------
    {
        const int Tn = a.n_total - a.n_clustered;
        const int t0 = (int)((int64_t)Tn * split / S), t1 = (int)((int64_t)Tn * (split + 1) / S);
        const T* Kt = reinterpret_cast<const T*>(a.K) + ubase;
        const T* Vt = reinterpret_cast<const T*>(a.V) + ubase;
        for (int base = t0 + wave * 8; base < t1; base += 32) {
            RowBuf<T> bf;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int i = base + u * 4 + rg;
                bf.ok[u] = i < t1;
                const int r = a.n_clustered + (bf.ok[u] ? i : t0);
                bf.k[u].load(Kt + (size_t)r * kHeadDim);
                bf.v[u].load(Vt + (size_t)r * kHeadDim);
            }
            exact_step<T, G>(st, qs, qscale, bf);
        }
    }
    // ---- the remaining removals (past the first step, second list) -------
    if (a.n_sub > 0)
        for (int base = sk0 + 32 + wave * 8; base < sk1; base += 32) {
            load_sub<T, G>(sub, a.sa, sids, unit, sk0, sk1, base, rg, li);
            absorb2<T, G, true>(st, sub.lg, sub.v);
        }
    if (a.n_sub > 1) {
        const int nk = a.sb.counts[unit * 4 + 1];
        const int k0 = (int)((int64_t)nk * split / S), k1 = (int)((int64_t)nk * (split + 1) / S);
        const int32_t* ids = a.sb.ids + (size_t)unit * a.sb.ids_stride;
        for (int base = k0 + wave * 8; base < k1; base += 32) {
            load_sub<T, G>(sub, a.sb, ids, unit, k0, k1, base, rg, li);
            absorb2<T, G, true>(st, sub.lg, sub.v);
        }
    }
    __syncthreads();  // the chunk staging (aliasing the reduction area) is consumed
    finish_partial<G>(st, s_red, a.part_ml, a.part_acc, unit, split, a.part_stride);
}

// Workgroup (split, unit).  The approximate term does not depend on the cut:
// split s also streams chunk s of the sources in a.pseudo (the coarse level,
// then the fine level; S is at least their chunk count) and folds it into its
// state.  The bf16 variants with up to 4 query heads per group are held to
// 128 registers so that 4 workgroups fit on a CU.
template <typename T, int G>
__global__ __launch_bounds__(256, (sizeof(T) == 2 && G <= 4) ? 4 : 1) void attend_kernel(AttendArgs a) {
    __shared__ __align__(16) char lds[attend_lds_bytes<G>()];
    attend_split<T, G>(a, blockIdx.x, blockIdx.y, lds);
}

// merge: one 128-thread workgroup per (unit, query head of the group) over the
// P partials of the unit, 8 partials loaded per round.
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_ml,
                                                    const float* __restrict__ part_acc, int G, int P, int Hkv,
                                                    float* __restrict__ out) {
    const int unit = blockIdx.x / G, g = blockIdx.x % G;
    const int dd = threadIdx.x;
    const size_t base = ((size_t)unit * G + g) * P;
    float M = -INFINITY;
    for (int s = 0; s < P; ++s) M = fmaxf(M, part_ml[(base + s) * 2]);
    float l = 0.f, acc = 0.f;
    if (M != -INFINITY) {
        for (int s0 = 0; s0 < P; s0 += 8) {
            float ml[8], lv[8], av[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int s = min(s0 + k, P - 1);
                ml[k] = part_ml[(base + s) * 2];
                lv[k] = part_ml[(base + s) * 2 + 1];
                av[k] = part_acc[(base + s) * kHeadDim + dd];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                if (s0 + k < P) {
                    const float w = __builtin_amdgcn_exp2f(ml[k] - M);
                    l = fmaf(lv[k], w, l);
                    acc = fmaf(av[k], w, acc);
                }
            }
        }
    }
    const int b = unit / Hkv, h = unit % Hkv;
    out[((size_t)b * Hkv * G + (size_t)h * G + g) * kHeadDim + dd] = l > 0.f ? acc / l : 0.f;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename T>
static hipError_t score_dispatch(int G, const ScoreArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: hipLaunchKernelGGL((score_kernel<T, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((score_kernel<T, 2>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((score_kernel<T, 4>), grid, dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((score_kernel<T, 8>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int score_chunks(int n_items) { return n_items > 0 ? (n_items + kScoreChunk - 1) / kScoreChunk : 0; }

hipError_t launch_score(int dtype, int G, const ScoreArgs& a, int units, hipStream_t st) {
    if (a.n_items <= 0) return hipSuccess;
    dim3 grid(score_chunks(a.n_items), units);
    return dtype == 1 ? score_dispatch<bf16_t>(G, a, grid, st) : score_dispatch<float>(G, a, grid, st);
}

hipError_t launch_select(const SelectArgs& a, int units, hipStream_t st) {
    if ((a.mask_bits + 31) / 32 > kMaskWords) return hipErrorInvalidValue;
    hipLaunchKernelGGL(select_kernel, dim3(units), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
static hipError_t attend_dispatch(int G, const AttendArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: hipLaunchKernelGGL((attend_kernel<T, 1>), grid, dim3(256), 0, st, a); break;
        case 2: hipLaunchKernelGGL((attend_kernel<T, 2>), grid, dim3(256), 0, st, a); break;
        case 4: hipLaunchKernelGGL((attend_kernel<T, 4>), grid, dim3(256), 0, st, a); break;
        case 8: hipLaunchKernelGGL((attend_kernel<T, 8>), grid, dim3(256), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_attend(int dtype, int G, const AttendArgs& a, int units, hipStream_t st) {
    if (a.S < 1 || a.S > a.part_stride || a.n_sub < 0 || a.n_sub > 2 || a.sel_stride < 1) return hipErrorInvalidValue;
    if (a.n_sub > 0 && a.sa.ids_stride != a.sel_stride) return hipErrorInvalidValue;
    if (a.n_pseudo < 0 || a.n_pseudo > 2) return hipErrorInvalidValue;
    int chunks = 0;
    for (int k = 0; k < a.n_pseudo; ++k) {
        if (a.pseudo[k].chunks != score_chunks(a.pseudo[k].n_items)) return hipErrorInvalidValue;
        chunks += a.pseudo[k].chunks;
    }
    if (chunks > a.S) return hipErrorInvalidValue;  // one chunk per split at most
    dim3 grid(a.S, units);
    return dtype == 1 ? attend_dispatch<bf16_t>(G, a, grid, st) : attend_dispatch<float>(G, a, grid, st);
}

hipError_t launch_merge(const float* part_ml, const float* part_acc, int units, int G, int P, int Hkv, float* out,
                        hipStream_t st) {
    hipLaunchKernelGGL(merge_kernel, dim3(units * G), dim3(kHeadDim), 0, st, part_ml, part_acc, G, P, Hkv, out);
    return hipGetLastError();
}

}  // namespace mpa
