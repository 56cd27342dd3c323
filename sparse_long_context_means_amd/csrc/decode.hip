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
//   score  -- s[c][g] = q_g . Kbar_c / sqrt(d), the group-mean ranking key and
//             the cluster size, packed per item for the cut;
//   select -- one workgroup per unit takes the budget cut (longest prefix of
//             the (key desc, id asc) order whose sizes fit the budget) with a
//             radix select, and writes the selected clusters (id, first member
//             position, prefix of member rows) and a bitmask of them;
//   attend -- split-K online softmax over the exact rows of the selected
//             clusters (gathered K/V), the unclustered tail and every
//             non-empty unselected cluster (logit s + ln n, value Vbar), in
//             base-2 exponent units, fp32 partials;
//   merge  -- log-sum-exp merge of the splits.
// Kernel boundaries carry the cross-workgroup dependencies: a device-scope
// fence per workgroup (write back + invalidate of an XCD's L2) serialises and
// costs far more than a launch on this chip.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;  // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int wave_exclusive_sum(int v, int& total) {
    const int inc = wave_inclusive_sum(v);
    total = lane_value(inc, kWave - 1);
    return inc - v;
}

// Largest k with pre[k] <= x, for pre[0] = 0 <= x < pre[n] (n >= 1).
__device__ __forceinline__ int upper_index(const int32_t* pre, int n, int x) {
    int lo = 0, hi = n;  // pre[lo] <= x < pre[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pre[mid] <= x) lo = mid;
        else hi = mid;
    }
    return lo;
}

// ---------------------------------------------------------------------------
// score: workgroup (chunk, unit) scores 256 items, 16 lanes per centroid row,
// 8 rows per lane group in flight, two passes.  Items are cluster ids, or the
// member rows of a previous selection (the fine clusters inside the coarse
// candidates of the two-level method).
// ---------------------------------------------------------------------------
constexpr int kScoreChunk = 256;  // items per workgroup (64 per wave)
constexpr int kListCap = 1024;    // selection-list entries staged in LDS

template <typename T, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    __shared__ int32_t s_pre[kListCap + 1];
    __shared__ int32_t s_off[kListCap];
    const int unit = blockIdx.y;
    int n = a.n_items;
    if (a.n_items_dev) n = min(n, a.n_items_dev[unit * 4]);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int i0 = blockIdx.x * kScoreChunk + wave * 64;
    if (blockIdx.x * kScoreChunk >= n) return;  // uniform across the workgroup

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
            for (int k = threadIdx.x; k <= nl; k += 256) {
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
    if (i0 >= n) return;

    const int b = unit / a.Hkv, h = unit % a.Hkv;
    QSlice<T> qv[G];
    const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
#pragma unroll
    for (int g = 0; g < G; ++g) qv[g].load(qb + (size_t)g * kHeadDim);
    const T* cu = reinterpret_cast<const T*>(a.cent) + (size_t)unit * a.cent_rows * kHeadDim + li * 8;
    const int32_t* szu = a.sizes + (size_t)unit * a.cent_rows;
#pragma unroll 1
    for (int half = 0; half < 2; ++half) {  // 2 x 8 rows per lane group in flight
        const int ib = i0 + half * 32;
        int cid[8];
        Slice8<T> row[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = ib + u * 4 + rg;
            const int ii = i < n ? i : i0;
            if (lpre) {
                const int k = upper_index(lpre, nl, ii);
                cid[u] = mem[loff[k] + ii - lpre[k]];
            } else {
                cid[u] = ii;
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) row[u].load(cu + (size_t)cid[u] * kHeadDim);
        int sz[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) sz[u] = li == 0 ? szu[cid[u]] : 0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = ib + u * 4 + rg;
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
                if (li == 0) a.rs_out[(size_t)unit * a.rs_stride + i] = make_int2(__float_as_int(r), sz[u]);
                if (a.ids_out && li == 15) a.ids_out[(size_t)unit * a.rs_stride + i] = cid[u];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// select: budget cut of one unit by one 256-thread workgroup.  Thread t owns
// items 8 t .. 8 t + 7 of each tile of 2048 (key and size in registers).
// Four 8-bit radix passes over the order-preserving key bits find the cut
// value: pass p adds the sizes of the items still matching the prefix into
// its own LDS histogram (all four are cleared up front, so a pass needs one
// barrier), then every wave scans that histogram from the top digit down to
// the budget left, and all reach the same digit.  Items above the cut value
// are selected; items equal to it are taken in item order while they fit.
// One workgroup scan places the selected items in item order.
// ---------------------------------------------------------------------------
constexpr int kSelItems = 8;                 // items per thread per tile
constexpr int kSelTileN = 256 * kSelItems;   // items per tile
constexpr int kMaskWords = 1024;             // LDS bitmask capacity (32768 ids)

struct SelItems {
    uint32_t key[kSelItems];
    int32_t sz[kSelItems];
};

__device__ __forceinline__ void load_items(const SelectArgs& a, int unit, int n, int base, SelItems& it) {
    const int2* rs = a.rs + (size_t)unit * a.rs_stride;
    const int t0 = base + threadIdx.x * kSelItems;
#pragma unroll
    for (int j = 0; j < kSelItems; ++j) {
        const int2 v = t0 + j < n ? rs[t0 + j] : make_int2(0, 0);
        it.key[j] = order_key(__int_as_float(v.x));
        it.sz[j] = v.y;
    }
}

__global__ __launch_bounds__(256) void select_kernel(SelectArgs a) {
    __shared__ int hist[4][256];
    __shared__ int scan_lds[16];
    __shared__ uint32_t s_mask[kMaskWords];
    const int unit = blockIdx.x;
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
    const int32_t* goff = a.offsets + (size_t)unit * a.off_stride;
    int32_t* sid = a.sel_ids + (size_t)unit * a.sel_stride;
    int32_t* soff = a.sel_off + (size_t)unit * a.sel_stride;
    int32_t* spre = a.sel_rowpre + (size_t)unit * (a.sel_stride + 1);
    int32_t* dbg = a.dbg_selected ? a.dbg_selected + (size_t)unit * a.dbg_stride : nullptr;
    int carry_rows = 0, carry_sel = 0, carry_tie = 0;
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
        if (!done) {
            // usually a single item carries the cut value: then no scan is needed
            const int holders = __syncthreads_count(tie_local > 0);
            if (holders > 1 || !resident) {
                int4 tt;
                run_tie += block256_exclusive_sum4(make_int4(tie_local, 0, 0, 0), tt, scan_lds).x;
                carry_tie += tt.x;
            }
        }
        uint32_t selbits = 0;
        int s_local = 0;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            const int sz = it.sz[j];
            const uint32_t u = it.key[j];
            bool sel;
            if (done) {
                sel = u >= prefix;
            } else {
                const bool tie = u == tau;
                sel = u > tau || (tie && run_tie + sz <= R);
                if (tie) run_tie += sz;
            }
            sel = sel && sz > 0;
            selbits |= (uint32_t)sel << j;
            s_local += sel;
        }
        // member rows of the selected items (offsets read only for those)
        int id[kSelItems], off[kSelItems], nr[kSelItems];
        int rows_local = 0;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            id[j] = t0 + j < n ? (gids ? gids[t0 + j] : t0 + j) : 0;
            off[j] = 0;
            nr[j] = 0;
            if ((selbits >> j) & 1u) {
                off[j] = goff[id[j]];
                nr[j] = goff[id[j] + 1] - off[j];
                rows_local += nr[j];
            }
        }
        int4 tot;
        const int4 ex = block256_exclusive_sum4(make_int4(s_local, rows_local, 0, 0), tot, scan_lds);
        int k = carry_sel + ex.x, ro = carry_rows + ex.y;
#pragma unroll
        for (int j = 0; j < kSelItems; ++j) {
            if ((selbits >> j) & 1u) {
                sid[k] = id[j];
                soff[k] = off[j];
                spre[k] = ro;
                ++k;
                ro += nr[j];
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
// attend: workgroup (split, unit), 4 waves, 16 lanes per row, 8 dims a lane.
// A row group (16 lanes) keeps its own online-softmax state (m, l, acc[8] per
// head) over the rows it visits, 2 rows per step with the next step's rows
// already in flight.  The running maximum is only raised when a logit exceeds
// it by more than 2^8 (every weight stays <= 256 in fp32), so rescaling is
// rare.  Exact rows: split s takes rows [E s / S, E (s + 1) / S) of the
// selected clusters' member rows (found by binary search of the row prefix).
// Approximated clusters: split s takes items [P s / S, P (s + 1) / S) of the
// cluster range and keeps the non-empty unselected ones (bitmask), compacted
// in LDS with their weights n 2^(lambda - M) (M the chunk maximum).
// ---------------------------------------------------------------------------
constexpr int kAttCap = 512;       // staged items per list and pass
constexpr float kLazyMax = 8.0f;   // base-2 headroom before the running max moves

template <int G>
struct SoftState {
    float m[G], l[G], acc[G][8];
};

// Adds 2 rows with base-2 logits lg[u][g] (-inf for an absent row).
template <typename T, int G>
__device__ __forceinline__ void absorb2(SoftState<G>& st, const float (&lg)[2][G], const Slice8<T> (&v)[2]) {
    float x0[8], x1[8];
    v[0].unpack(x0);
    v[1].unpack(x1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mx = fmaxf(lg[0][g], lg[1][g]);
        if (mx == -INFINITY) continue;
        if (mx > st.m[g] + kLazyMax) {  // rare: raise the reference maximum
            const float sc = __builtin_amdgcn_exp2f(st.m[g] - mx);
            st.l[g] *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[g][e] *= sc;
            st.m[g] = mx;
        }
        const float p0 = __builtin_amdgcn_exp2f(lg[0][g] - st.m[g]);
        const float p1 = __builtin_amdgcn_exp2f(lg[1][g] - st.m[g]);
        st.l[g] += p0 + p1;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(p1, x1[e], fmaf(p0, x0[e], st.acc[g][e]));
    }
}

// Merge another partial state (om, ol, oacc) into st.
template <int G>
__device__ __forceinline__ void merge_state(SoftState<G>& st, const float* om, const float* ol, const float (*oacc)[8]) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = fmaxf(st.m[g], om[g]);
        if (M == -INFINITY) continue;
        const float wa = __builtin_amdgcn_exp2f(st.m[g] - M);
        const float wb = __builtin_amdgcn_exp2f(om[g] - M);
        st.l[g] = st.l[g] * wa + ol[g] * wb;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] = st.acc[g][e] * wa + oacc[g][e] * wb;
        st.m[g] = M;
    }
}

template <typename T>
struct RowBuf {
    Slice8<T> k[2], v[2];
    bool ok[2];
};

// Loads rows it * 32 + wave * 8 + u * 4 + rg (u = 0, 1) of a staged list.
template <typename T>
__device__ __forceinline__ void load_rows(RowBuf<T>& bf, const int32_t* s_row, int cnt, int it, int wave, int rg,
                                          const T* Kx, const T* Vx) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = it * 32 + wave * 8 + u * 4 + rg;
        bf.ok[u] = i < cnt;
        const int r = s_row[bf.ok[u] ? i : 0];
        bf.k[u].load(Kx + (size_t)r * kHeadDim);
        bf.v[u].load(Vx + (size_t)r * kHeadDim);
    }
}

template <typename T, int G>
__device__ __forceinline__ void exact_step(SoftState<G>& st, const QSlice<T> (&qs)[G], float qscale,
                                           const RowBuf<T>& bf) {
    float lg[2][G];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float d = row16_sum(dot8(qs[g], bf.k[u])) * qscale;
            lg[u][g] = bf.ok[u] ? d : -INFINITY;
        }
    absorb2<T, G>(st, lg, bf.v);
}

template <typename T>
struct PseudoBuf {
    Slice8<T> v[2];
    bool ok[2];
    int i[2];
};

template <typename T>
__device__ __forceinline__ void load_pseudo(PseudoBuf<T>& bf, const int32_t* s_pid, int cnt, int it, int wave, int rg,
                                            const T* vbar) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = it * 32 + wave * 8 + u * 4 + rg;
        bf.ok[u] = i < cnt;
        bf.i[u] = bf.ok[u] ? i : 0;
        bf.v[u].load(vbar + (size_t)s_pid[bf.i[u]] * kHeadDim);
    }
}

// Adds 2 approximated clusters: staged weights (relative to the chunk
// reference) times the row group's factor f.
template <typename T, int G>
__device__ __forceinline__ void pseudo_step(SoftState<G>& st, const float (*s_w)[G], const float (&f)[G],
                                            const PseudoBuf<T>& bf) {
    float x0[8], x1[8];
    bf.v[0].unpack(x0);
    bf.v[1].unpack(x1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float p0 = bf.ok[0] ? s_w[bf.i[0]][g] * f[g] : 0.f;
        const float p1 = bf.ok[1] ? s_w[bf.i[1]][g] * f[g] : 0.f;
        st.l[g] += p0 + p1;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(p1, x1[e], fmaf(p0, x0[e], st.acc[g][e]));
    }
}

// Stages exact rows [c0, c0 + cnt) of the unit's selection: row i belongs to
// selected cluster k with pre[k] <= i < pre[k + 1] and sits at member position
// off[k] + i - pre[k] (through token ids when rows are gathered from K/V).
__device__ __forceinline__ void stage_exact(int32_t* s_row, const int32_t* pre, const int32_t* off, int nsel,
                                            const int32_t* tids, int c0, int cnt) {
    for (int i = threadIdx.x; i < cnt; i += 256) {
        const int r = c0 + i;
        const int k = upper_index(pre, nsel, r);
        const int pos = off[k] + r - pre[k];
        s_row[i] = tids ? tids[pos] : pos;
    }
}

// Stages the approximated clusters among items [c0, c0 + cnt) (cnt <= 512)
// of a source: non-empty and not selected, compacted in item order; for each,
// per head the weight n * 2^(lambda - M) with lambda = s * log2(e) (base-2
// logit) and M the chunk's largest log2(n) + lambda, left in s_pm[g].
// Returns the number staged.  Ends with a barrier.
template <int G>
__device__ __forceinline__ int stage_pseudo(int32_t* s_pid, float (*s_w)[G], float* s_pm, float (*s_wmax)[G],
                                            int* s_cnt, const PseudoSrc& ps, int unit, int c0, int cnt) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int32_t* ids = ps.ids ? ps.ids + (size_t)unit * ps.ids_stride : nullptr;
    const uint32_t* msk = ps.selmask + (size_t)unit * ps.mask_stride;
    const float* su = ps.s + (size_t)unit * ps.rows * G;
    const int32_t* szu = ps.sizes + (size_t)unit * ps.rows;
    float lg[2][G];
    int cid[2];
    bool keep[2];
    float mx[G];
#pragma unroll
    for (int g = 0; g < G; ++g) mx[g] = -INFINITY;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int i = tid + 256 * k;
        keep[k] = false;
        cid[k] = 0;
        if (i < cnt) {
            const int c = ids ? ids[c0 + i] : c0 + i;
            const int n = szu[c];
            cid[k] = c;
            keep[k] = n > 0 && !((msk[c >> 5] >> (c & 31)) & 1u);
            if (keep[k]) {
                const float ln2n = __builtin_amdgcn_logf((float)n);  // log2(n)
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    lg[k][g] = fmaf(su[(size_t)c * G + g], kLog2e, ln2n);
                    mx[g] = fmaxf(mx[g], lg[k][g]);
                }
            }
        }
    }
    // per-wave maxima and kept counts; one barrier
    const uint64_t b0 = __ballot(keep[0]), b1 = __ballot(keep[1]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float m = mx[g];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, shfl_xor_f(m, o));
        if (lane == 0) s_wmax[wave][g] = m;
    }
    if (lane == 0) {
        s_cnt[wave] = __popcll(b0);
        s_cnt[4 + wave] = __popcll(b1);
    }
    __syncthreads();
#pragma unroll
    for (int g = 0; g < G; ++g)
        mx[g] = fmaxf(fmaxf(s_wmax[0][g], s_wmax[1][g]), fmaxf(s_wmax[2][g], s_wmax[3][g]));
#pragma unroll
    for (int g = 0; g < G; ++g)
        if (tid == g) s_pm[g] = mx[g];
    // item order: k = 0 items (threads 0..255) first, then k = 1
    int base0 = 0, base1 = 0, total = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        base0 += w < wave ? s_cnt[w] : 0;
        total += s_cnt[w];
    }
    base1 = total;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        base1 += w < wave ? s_cnt[4 + w] : 0;
        total += s_cnt[4 + w];
    }
    const uint64_t below = (1ull << lane) - 1;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (keep[k]) {
            const int slot = (k == 0 ? base0 + __popcll(b0 & below) : base1 + __popcll(b1 & below));
            s_pid[slot] = cid[k];
#pragma unroll
            for (int g = 0; g < G; ++g) s_w[slot][g] = __builtin_amdgcn_exp2f(lg[k][g] - mx[g]);
        }
    }
    __syncthreads();
    return total;
}

template <typename T, int G>
__global__ __launch_bounds__(256) void attend_kernel(AttendArgs a) {
    __shared__ int32_t s_row[kAttCap];
    __shared__ int32_t s_pid[kAttCap];
    __shared__ float s_w[kAttCap][G];
    __shared__ float s_pm[G];
    __shared__ float s_wmax[4][G];
    __shared__ int s_cnt[8];
    __shared__ int32_t s_pre[kListCap + 1];
    __shared__ int32_t s_off[kListCap];
    __shared__ float s_red[4][G][kHeadDim + 2];

    const int split = blockIdx.x, unit = blockIdx.y;
    const int S = a.S;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    const float qscale = kInvSqrtD * kLog2e;

    // selection of the unit: member-row prefix and first member of each
    // selected cluster (staged when small enough)
    const int E = a.counts[unit * 4];
    const int nsel = a.counts[unit * 4 + 1];
    const int e0 = (int)((int64_t)E * split / S), e1 = (int)((int64_t)E * (split + 1) / S);
    const int32_t* gpre = a.sel_rowpre + (size_t)unit * (a.sel_stride + 1);
    const int32_t* goff = a.sel_off + (size_t)unit * a.sel_stride;
    const int32_t* pre = gpre;
    const int32_t* off = goff;
    if (nsel <= kListCap) {
        for (int k = tid; k <= nsel; k += 256) {
            s_pre[k] = gpre[k];
            if (k < nsel) s_off[k] = goff[k];
        }
        pre = s_pre;
        off = s_off;
    }
    const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
    QSlice<T> qs[G];
#pragma unroll
    for (int g = 0; g < G; ++g) qs[g].load(qb + (size_t)g * kHeadDim);
    SoftState<G> st;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        st.m[g] = -INFINITY;
        st.l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) st.acc[g][e] = 0.f;
    }
    const size_t ubase = (size_t)unit * a.Nmax * kHeadDim + li * 8;
    const T* Kx = reinterpret_cast<const T*>(a.Kx) + ubase;
    const T* Vx = reinterpret_cast<const T*>(a.Vx) + ubase;
    const int32_t* tids = a.token_ids ? a.token_ids + (size_t)unit * a.Nmax : nullptr;
    __syncthreads();

    // ---- exact rows of selected clusters -------------------------------
    for (int c0 = e0; c0 < e1; c0 += kAttCap) {
        const int cnt = min(kAttCap, e1 - c0);
        if (c0 != e0) __syncthreads();
        stage_exact(s_row, pre, off, nsel, tids, c0, cnt);
        __syncthreads();
        const int steps = (cnt + 31) / 32;
        RowBuf<T> A, B;
        if (steps > 0) load_rows<T>(A, s_row, cnt, 0, wave, rg, Kx, Vx);
        for (int it = 0; it < steps; it += 2) {
            if (it + 1 < steps) load_rows<T>(B, s_row, cnt, it + 1, wave, rg, Kx, Vx);
            exact_step<T, G>(st, qs, qscale, A);
            if (it + 1 < steps) {
                if (it + 2 < steps) load_rows<T>(A, s_row, cnt, it + 2, wave, rg, Kx, Vx);
                exact_step<T, G>(st, qs, qscale, B);
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
    // ---- approximated clusters: logit s + ln n, value Vbar ----------------
#pragma unroll 1
    for (int which = 0; which < a.n_pseudo; ++which) {
        const PseudoSrc& ps = which == 0 ? a.pa : a.pb;
        const int P = ps.n_dev ? min(ps.n_host, ps.n_dev[unit * 4]) : ps.n_host;
        const int p0 = (int)((int64_t)P * split / S), p1 = (int)((int64_t)P * (split + 1) / S);
        const T* vbar = reinterpret_cast<const T*>(ps.vbar) + (size_t)unit * ps.rows * kHeadDim + li * 8;
        for (int c0 = p0; c0 < p1; c0 += kAttCap) {
            __syncthreads();
            const int cnt = stage_pseudo<G>(s_pid, s_w, s_pm, s_wmax, s_cnt, ps, unit, c0, min(kAttCap, p1 - c0));
            // move this row group's state to reference max(m, M) once; the
            // staged weights are relative to M
            float f[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float M = s_pm[g];
                if (M > st.m[g]) {
                    const float sc = __builtin_amdgcn_exp2f(st.m[g] - M);
                    st.l[g] *= sc;
#pragma unroll
                    for (int e = 0; e < 8; ++e) st.acc[g][e] *= sc;
                    st.m[g] = M;
                }
                f[g] = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - st.m[g]);
            }
            const int steps = (cnt + 31) / 32;
            PseudoBuf<T> A, B;
            if (steps > 0) load_pseudo<T>(A, s_pid, cnt, 0, wave, rg, vbar);
            for (int it = 0; it < steps; it += 2) {
                if (it + 1 < steps) load_pseudo<T>(B, s_pid, cnt, it + 1, wave, rg, vbar);
                pseudo_step<T, G>(st, s_w, f, A);
                if (it + 1 < steps) {
                    if (it + 2 < steps) load_pseudo<T>(A, s_pid, cnt, it + 2, wave, rg, vbar);
                    pseudo_step<T, G>(st, s_w, f, B);
                }
            }
        }
    }

    // ---- merge the 4 row groups of the wave, then the 4 waves --------------
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
    // thread -> (g, dim) pairs; waves merged in order 0..3
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
        const size_t pidx = ((size_t)unit * G + g) * S + split;
        a.part_acc[pidx * kHeadDim + dd] = acc;
        if (dd == 0) {
            a.part_ml[pidx * 2] = M;
            a.part_ml[pidx * 2 + 1] = l;
        }
    }
}

// merge: one 128-thread workgroup per (unit, query head of the group).
__global__ __launch_bounds__(128) void merge_kernel(const float* __restrict__ part_ml,
                                                    const float* __restrict__ part_acc, int G, int S, int Hkv,
                                                    float* __restrict__ out) {
    const int unit = blockIdx.x / G, g = blockIdx.x % G;
    const int dd = threadIdx.x;
    const size_t base = ((size_t)unit * G + g) * S;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, part_ml[(base + s) * 2]);
    float l = 0.f, acc = 0.f;
    if (M != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float w = __builtin_amdgcn_exp2f(part_ml[(base + s) * 2] - M);
            l = fmaf(part_ml[(base + s) * 2 + 1], w, l);
            acc = fmaf(part_acc[(base + s) * kHeadDim + dd], w, acc);
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

hipError_t launch_score(int dtype, int G, const ScoreArgs& a, int units, hipStream_t st) {
    if (a.n_items <= 0) return hipSuccess;
    dim3 grid((a.n_items + kScoreChunk - 1) / kScoreChunk, units);
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
    dim3 grid(a.S, units);
    return dtype == 1 ? attend_dispatch<bf16_t>(G, a, grid, st) : attend_dispatch<float>(G, a, grid, st);
}

hipError_t launch_merge(const float* part_ml, const float* part_acc, int units, int G, int S, int Hkv, float* out,
                        hipStream_t st) {
    hipLaunchKernelGGL(merge_kernel, dim3(units * G), dim3(kHeadDim), 0, st, part_ml, part_acc, G, S, Hkv, out);
    return hipGetLastError();
}

}  // namespace mpa
