// hier.hip -- one decode step of the hierarchical method for a (sequence, KV
// head) unit in one launch: R workgroups of 512 threads per unit.
//
// Pages: atlas.scime.ai summary, "Approach" (the hierarchical variant: coarse
// centroids over the fine ones, lookup and approximation at two levels) and
// opening sentence (exact attention on the top-scoring clusters, centroid
// terms for the rest).
//
// Every workgroup of a unit takes the same two cuts with the same operations:
//   1. keys of all coarse clusters: it scores its share on the matrix cores
//      and takes the other shares' keys from the other workgroups as tagged
//      64-bit words (or scores them itself when a partner is late: the same
//      bits); the key is the group mean;
//   2. the coarse cut under the candidate budget (candidates);
//   3. the candidates' non-empty fine clusters, listed by coarse id, then in
//      member order;
//   4. scores of those fine clusters; the fine cut under the token budget,
//      in (key desc, fine id asc) order;
// then takes its share of the work:
//   5. approximate terms: its share of the coarse clusters that are not
//      candidates, and of the candidates' fine clusters that were not
//      selected (n exp(s) on the value centroid, per query head);
//   6. exact rows: its share of the selected fine clusters' members followed
//      by the unclustered tail;
//   7. the partials of the workgroups are merged by the last one to finish,
//      through tagged 64-bit words as in unit.hip.
#include <math.h>

#include "attn.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

constexpr int kHThreads = 512;
constexpr int kHWaves = kHThreads / kWave;  // 8
constexpr int kHRowBatch = 1024;            // staged exact rows per pass
constexpr int kHScoreDepth = 2;             // score steps in flight per wave (4 measured slower)
constexpr int kHExactDepth = 2;             // exact-row steps (16 rows) in flight per wave
constexpr int kHCoarseAhead = 1;            // coarse value rows per row group loaded during the key exchange
constexpr int kHFineAhead = 1;              // fine value rows per row group loaded with the fine scores
// Waits on the other workgroups of a unit, in ticks of the 100 MHz constant
// clock: for their coarse keys (then the workgroup scores them itself) and
// for the partial words of workgroups that have already counted in.
constexpr uint64_t kHExchangeWaitTicks = 2000;
constexpr uint64_t kHPartialWaitTicks = 100000;

// Exclusive scan of one counter over the workgroup in thread order (`lds`:
// kHWaves ints); the total in tot.
__device__ __forceinline__ int block_exclusive_sum(int v, int& tot, int* lds) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int inc = wave_inclusive_sum(v);
    if (lane == kWave - 1) lds[wave] = inc;
    lds_barrier();
    int base = 0, t = 0;
#pragma unroll
    for (int w = 0; w < kHWaves; ++w) {
        const int x = lds[w];
        if (w < wave) base += x;
        t += x;
    }
    lds_barrier();  // lds may be reused right after
    tot = t;
    return base + inc - v;
}

// Exclusive scans of two counters over the workgroup in thread order, with
// one barrier each way (`lds`: 2 kHWaves ints); the totals in tot.
__device__ __forceinline__ int2 block_exclusive_sum2(int2 v, int2& tot, int* lds) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ix = wave_inclusive_sum(v.x), iy = wave_inclusive_sum(v.y);
    if (lane == kWave - 1) {
        lds[2 * wave] = ix;
        lds[2 * wave + 1] = iy;
    }
    lds_barrier();
    int bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
    for (int w = 0; w < kHWaves; ++w) {
        const int x = lds[2 * w], y = lds[2 * w + 1];
        if (w < wave) {
            bx += x;
            by += y;
        }
        tx += x;
        ty += y;
    }
    lds_barrier();  // lds may be reused right after
    tot = make_int2(tx, ty);
    return make_int2(bx + ix - v.x, by + iy - v.y);
}

// Budget cut over n items by the whole workgroup: the longest prefix of the
// non-empty items in (key desc, id asc) order whose sizes sum to at most
// `budget`.  A pass over equal-width value bins usually settles it; else four
// 8-bit radix passes over the order-preserving key bits of the items still
// open, weighted by size, find the cut value, and items at it are taken in id
// order while they fit.  Thread t owns items ITEMS t .. ITEMS t + ITEMS - 1;
// bit j of the result is item ITEMS t + j.  key(i), size(i), id(i) read item
// i (i < n); id orders items with equal keys.
template <int ITEMS, typename KeyF, typename SizeF, typename IdF>
__device__ __forceinline__ uint32_t block_cut(KeyF key_of, SizeF size_of, IdF id_of, int n, int budget,
                                              int (*hist)[256], int* scan) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    uint32_t key[ITEMS];
    float kf[ITEMS];
    int isz[ITEMS];
    uint32_t act = 0, bits = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = tid * ITEMS + j;
        kf[j] = i < n ? key_of(i) : 0.f;
        key[j] = order_key(kf[j]);
        isz[j] = i < n ? size_of(i) : 0;
        act |= (uint32_t)(isz[j] > 0) << j;
    }
    int Rb = budget;
    if (range_cut<kHWaves, ITEMS>(kf, key, isz, [&](int j) { return id_of(tid * ITEMS + j); }, Rb, act, bits,
                                  reinterpret_cast<unsigned long long*>(&hist[0][0]), reinterpret_cast<float*>(scan),
                                  []() { lds_barrier(); }))
        return bits;
    // (uniform, rare) exact radix passes over the open items
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) isz[j] = ((act >> j) & 1u) ? isz[j] : 0;
    lds_barrier();  // the first pass's histogram is read
    for (int k = tid; k < 4 * 256; k += kHThreads) reinterpret_cast<int*>(hist)[k] = 0;
    lds_barrier();
    uint32_t prefix = 0, pmask = 0;
    bool done = false;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int shift = 24 - 8 * p;
#pragma unroll
        for (int j = 0; j < ITEMS; ++j)
            if (isz[j] > 0 && (key[j] & pmask) == prefix) atomicAdd(&hist[p][(key[j] >> shift) & 255u], isz[j]);
        lds_barrier();
        int v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = hist[p][255 - (4 * lane + q)];
        int total;
        int run = wave_exclusive_sum(v[0] + v[1] + v[2] + v[3], total);
        if (total <= Rb) {  // the same in every wave: every candidate left fits
            done = true;
            break;
        }
        int found = -1, cum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            if (found < 0 && run <= Rb && Rb < run + v[q]) {
                found = 255 - (4 * lane + q);
                cum = run;
            }
            run += v[q];
        }
        const uint64_t bal = __ballot(found >= 0);
        const int src = __ffsll((long long)bal) - 1;
        const int digit = lane_value(found, src);
        Rb -= lane_value(cum, src);
        prefix |= (uint32_t)digit << shift;
        pmask |= 0xFFu << shift;
    }
    if (done) {
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) bits |= (uint32_t)(isz[j] > 0 && key[j] >= prefix) << j;
        return bits;
    }
    // items at the cut value, in id order while they fit: an item's running
    // sum is the sizes of the tied items with lower ids (ties are rare, so
    // each tied item scans all items; an item at the cut value is open, as
    // the taken items' keys lie above every open key and the dropped ones'
    // below)
    int ties = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) ties += isz[j] > 0 && key[j] == prefix;
    int tt;
    block_exclusive_sum(ties, tt, scan);  // tt: tied items in the workgroup
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        bool sel = isz[j] > 0 && key[j] > prefix;
        if (isz[j] > 0 && key[j] == prefix) {
            int run = 0;
            if (tt > 1) {
                const int me = id_of(tid * ITEMS + j);
                for (int i = 0; i < n; ++i) {
                    const int s = size_of(i);
                    if (s > 0 && id_of(i) < me && order_key(key_of(i)) == prefix) run += s;
                }
            }
            sel = run + isz[j] <= Rb;
        }
        bits |= (uint32_t)sel << j;
    }
    return bits;
}

// LDS layout (bytes).  Regions reused once their phase is over are noted.
template <int G>
struct HierLds {
    static constexpr int ckey = 0;                               // float [MaxD]: coarse keys; then int
                                                                 // [MaxD] candidate prefix; then int
                                                                 // [MaxF] selected list (spans csz too)
    static constexpr int csz = ckey + kHierMaxD * 4;             // int [MaxD]: coarse sizes
    static constexpr int cmask = csz + kHierMaxD * 4;            // uint32 [MaxD / 32]: candidates
    static constexpr int fid = cmask + kHierMaxD / 8;            // int [MaxF]: candidates' fine ids
    static constexpr int fkey = fid + kHierMaxF * 4;             // float [MaxF]: fine keys
    static constexpr int fsz = fkey + kHierMaxF * 4;             // int [MaxF]: fine sizes
    static constexpr int fmask = fsz + kHierMaxF * 4;            // uint32 [MaxF / 32]: selected
    static constexpr int spre = fmask + kHierMaxF / 8;           // int [MaxF + 4]: candidate coarse
                                                                 // ids; then selected-row prefix
    static constexpr int lg = spre + (kHierMaxF + 4) * 4;        // float [MaxShare][G]
    static constexpr int hist = (lg + kHierMaxShare * G * 4 + 15) / 16 * 16;  // int [4][256]
    static constexpr int scan = hist + 4 * 256 * 4;              // int [64]
    static constexpr int misc = scan + 64 * 4;                   // int [16]
    static constexpr int gmax = misc + 16 * 4;                   // float [waves][G]
    static constexpr int pexp = gmax + kHWaves * G * 4;         // float [waves][16][G]
    static constexpr int row = pexp + kHWaves * 16 * G * 4;     // int [RowBatch]
    static constexpr int foff = row + kHRowBatch * 4;            // int [MaxF]: candidates' member starts
    static constexpr int bytes = foff + kHierMaxF * 4;
    static constexpr int red = fid;                              // float [waves][G][d + 2], after the
                                                                 // exact rows (spans fid, fkey)
    static_assert(kHWaves * G * (kHeadDim + 2) * 4 <= 2 * kHierMaxF * 4, "reduction region");
    static_assert(hist % 16 == 0 && 256 * 8 + kRankCap * 16 <= 4 * 256 * 4, "value-bin pass in the histogram");
    static_assert(2 * kHWaves + 1 <= 64, "value-bin pass in the scan words");
};

template <int G>
__global__ __launch_bounds__(kHThreads) void hier_decode_kernel(HierArgs a) {
    using L = HierLds<G>;
    __shared__ __align__(16) char lds[L::bytes];
    float* s_ckey = reinterpret_cast<float*>(lds + L::ckey);
    int32_t* s_cpre = reinterpret_cast<int32_t*>(lds + L::ckey);  // after the coarse cut
    int32_t* s_sid = reinterpret_cast<int32_t*>(lds + L::ckey);   // after the fine cut
    int32_t* s_csz = reinterpret_cast<int32_t*>(lds + L::csz);
    uint32_t* s_cmask = reinterpret_cast<uint32_t*>(lds + L::cmask);
    int32_t* s_fid = reinterpret_cast<int32_t*>(lds + L::fid);
    float* s_fkey = reinterpret_cast<float*>(lds + L::fkey);
    int32_t* s_fsz = reinterpret_cast<int32_t*>(lds + L::fsz);
    uint32_t* s_fmask = reinterpret_cast<uint32_t*>(lds + L::fmask);
    int32_t* s_ccand = reinterpret_cast<int32_t*>(lds + L::spre);  // candidates' member starts, before the fine cut
    int32_t* s_spre = reinterpret_cast<int32_t*>(lds + L::spre);
    float(*s_lg)[G] = reinterpret_cast<float(*)[G]>(lds + L::lg);
    int(*hist)[256] = reinterpret_cast<int(*)[256]>(lds + L::hist);
    int* s_scan = reinterpret_cast<int*>(lds + L::scan);
    int* s_misc = reinterpret_cast<int*>(lds + L::misc);
    float(*s_gmax)[G] = reinterpret_cast<float(*)[G]>(lds + L::gmax);
    float* s_p = reinterpret_cast<float*>(lds + L::pexp);
    int32_t* s_row = reinterpret_cast<int32_t*>(lds + L::row);
    int32_t* s_foff = reinterpret_cast<int32_t*>(lds + L::foff);
    float(*s_red)[G][kHeadDim + 2] = reinterpret_cast<float(*)[G][kHeadDim + 2]>(lds + L::red);

    const int unit = blockIdx.x, rep = blockIdx.y, R = gridDim.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    const int D = a.D, C = a.C;
    // the call's tag of the unit's exchange words: one more than the tag of
    // its last decode (0 is never a tag: a zeroed word matches no call)
    uint32_t tag = a.xepoch[unit] + 1u;
    if (tag == 0u) tag = 1u;
    const bf16_t* qg = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim;
    const bf16_t* ck = reinterpret_cast<const bf16_t*>(a.ckbar) + (size_t)unit * a.Dmax * kHeadDim;
    const bf16_t* fk = reinterpret_cast<const bf16_t*>(a.kbar) + (size_t)unit * a.Cmax * kHeadDim;
    const int32_t* csizes = a.csizes + (size_t)unit * a.Dmax;
    const int32_t* coffs = a.coffsets + (size_t)unit * (a.Dmax + 1);
    const int32_t* cmem = a.cmembers + (size_t)unit * a.Cmax;
    const int32_t* fsizes = a.sizes + (size_t)unit * a.Cmax;
    const int32_t* foffs = a.offsets + (size_t)unit * (a.Cmax + 1);
    const bool dbg = rep == 0;

    // optional inspection: zeros first (the cuts set their ones after a
    // barrier that orders global memory)
    if (dbg && a.dbg_selected)
        for (int i = tid; i < C; i += kHThreads) a.dbg_selected[(size_t)unit * C + i] = 0;

    QOperand qop;
    load_qop<G>(qop, qg, lane);
    float lgmax = -INFINITY;  // the lane's maximum share logit (head li)

    // Scores of items [lo, hi): row(i) is the centroid row of item i; the
    // ranking key of item i goes to keys[i] (if keys), the base-2 logit
    // s log2(e) + log2(size) of items of [s0, s1) to s_lg[i - s0 + lg0].
    // Lane l loads row l % 16 of its wave's 16; the waves interleave.  pre()
    // runs once the first rows are in flight (it may end with a barrier).
    // The same item gets the same bits whichever pass scores it.
    auto score_items = [&](int lo, int hi, auto row_of, auto size_of, float* keys, int s0, int s1, int lg0,
                           auto pre) {
        if (hi <= lo) {  // (uniform) row lo exists only for hi > lo
            pre();
            return;
        }
        const int steps = (hi - lo + 16 * kHWaves - 1) / (16 * kHWaves);
        auto base = [&](int step) { return lo + step * 16 * kHWaves + wave * 16; };
        Slice8<bf16_t> ring[kHScoreDepth][4];
#pragma unroll
        for (int j = 0; j < kHScoreDepth; ++j) {
            const int i = base(j) + li;
            load_row_blocks(ring[j], row_of(i < hi ? i : lo), lane);
            __builtin_amdgcn_sched_barrier(0);
        }
        pre();
        auto consume = [&](const Slice8<bf16_t> (&r)[4], int s) {
            const f32x4v d = mfma_scores(r, qop);
            const int cb = base(s) + 4 * rg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = d[e] * kInvSqrtD;
                const float key = head_mean<G>(sv);
                const int i = cb + e;
                if (i < hi) {
                    if (li == 0 && keys) keys[i] = key;
                    if (li < G && i >= s0 && i < s1) {
                        const int sz = size_of(i);
                        const float lgv = sz > 0 ? fmaf(sv, kLog2e, log2_count(sz)) : -INFINITY;
                        s_lg[i - s0 + lg0][li] = lgv;
                        lgmax = fmaxf(lgmax, lgv);
                    }
                }
            }
        };
        // the last group is consumed without loading rows past the end, so
        // nothing is left in flight for the next phase's first wait
        int it = 0;
        for (; it + kHScoreDepth < steps; it += kHScoreDepth) {
#pragma unroll
            for (int j = 0; j < kHScoreDepth; ++j) {
                consume(ring[j], it + j);
                const int i = base(it + j + kHScoreDepth) + li;
                load_row_blocks(ring[j], row_of(i < hi ? i : lo), lane);
                __builtin_amdgcn_sched_barrier(0);  // keep the ring order
            }
        }
#pragma unroll
        for (int j = 0; j < kHScoreDepth; ++j) consume(ring[j], it + j);
    };

    // ---- 1. coarse scores.  With several workgroups each scores its share
    //      [cs0, cs1) and takes the others' keys as 64-bit words (call tag
    //      << 32 | key bits) that every workgroup stores into each other's
    //      slot; a word counts once it carries this call's tag, so no fence
    //      orders the words and words of earlier calls need no clearing.  If
    //      a word is still missing after kHExchangeWaitTicks (a partner not
    //      yet running), the workgroup scores every coarse cluster itself,
    //      which gives the same keys.  The coarse sizes go out ahead of the
    //      rows, as unconditional loads (clamped index), and reach LDS while
    //      the first rows are in flight.
    constexpr int kCItems = kHierMaxD / kHThreads;
    int csz_r[kCItems];
#pragma unroll
    for (int j = 0; j < kCItems; ++j) csz_r[j] = csizes[min(tid + j * kHThreads, D - 1)];
    // member ranges of the thread's coarse clusters in the cut's item order
    // (items kCItems t .. kCItems t + kCItems - 1), in flight with the rows
    int cof_r[kCItems + 1];
#pragma unroll
    for (int j = 0; j <= kCItems; ++j) cof_r[j] = coffs[min(tid * kCItems + j, D)];
    const int cs0 = (int)((int64_t)D * rep / R), cs1 = (int)((int64_t)D * (rep + 1) / R);
    const bool xchg = R > 1 && a.rescore != 1;
    auto crow = [&](int i) { return ck + (size_t)i * kHeadDim; };
    auto csize = [&](int i) { return s_csz[i]; };
    score_items(xchg ? cs0 : 0, xchg ? cs1 : D, crow, csize, s_ckey, cs0, cs1, 0, [&]() {
#pragma unroll
        for (int j = 0; j < kCItems; ++j)
            if (tid + j * kHThreads < D) s_csz[tid + j * kHThreads] = csz_r[j];
        for (int i = tid; i < kHierMaxD / 32; i += kHThreads) s_cmask[i] = 0u;
        for (int i = tid; i < kHierMaxF / 32; i += kHThreads) s_fmask[i] = 0u;
        if (tid == 0) s_misc[1] = 0;
        lds_barrier();
    });
    lds_barrier();
    // the share's first coarse value rows (row group rgi takes items rgi +
    // 32 j of the share, the order of the approximate-term pass below) go out
    // now, the candidates among them too (their weight is 0), and are added
    // after the fine cut: they arrive while the partners' keys are awaited
    // (a wave's loads complete in issue order, so a later load's wait covers
    // them too) and the lookup in between reads little
    const int dsh = cs1 - cs0;  // coarse share logits at s_lg[0 .. dsh)
    const int rgi = wave * 4 + rg;
    constexpr int kPass = 4 * kHWaves;
    const bf16_t* cv = reinterpret_cast<const bf16_t*>(a.cvbar) + (size_t)unit * a.Dmax * kHeadDim + li * 8;
    Slice8<bf16_t> pv[kHCoarseAhead];
    if (a.pseudo && dsh > 0) {  // (uniform)
#pragma unroll
        for (int j = 0; j < kHCoarseAhead; ++j) pv[j].load(cv + (size_t)(cs0 + min(rgi + j * kPass, dsh - 1)) * kHeadDim);
    }
    if (xchg) {
        const uint64_t tagw = (uint64_t)tag << 32;
        uint64_t* xu = a.xch + (size_t)unit * R * a.Dmax;
        for (int i = cs0 + tid; i < cs1; i += kHThreads) {
            const uint64_t w = tagw | __float_as_uint(s_ckey[i]);
            for (int r2 = 0; r2 < R; ++r2)
                if (r2 != rep)
                    __hip_atomic_store(xu + (size_t)r2 * a.Dmax + i, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        bool miss = a.rescore == 2;  // 2: as if the other keys never came
        if (!miss) {
            const uint64_t* slot = xu + (size_t)rep * a.Dmax;
            uint64_t w[kCItems];
#pragma unroll
            for (int q = 0; q < kCItems; ++q)  // unconditional (clamped): exact wait counts
                w[q] = __hip_atomic_load(slot + min(tid + q * kHThreads, D - 1), __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT);
            // stale words are read again in one batch per round (one trip to
            // memory a round), for a bounded time
            const uint64_t t0 = wall_clock64();
            for (;;) {
                bool stale = false;
#pragma unroll
                for (int q = 0; q < kCItems; ++q) {
                    const int i = tid + q * kHThreads;
                    stale = stale || (i < D && (i < cs0 || i >= cs1) && (uint32_t)(w[q] >> 32) != tag);
                }
                if (!stale) break;
                if (wall_clock64() - t0 > kHExchangeWaitTicks) {
                    miss = true;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
#pragma unroll
                for (int q = 0; q < kCItems; ++q) {
                    const int i = tid + q * kHThreads;
                    if (i < D && (i < cs0 || i >= cs1) && (uint32_t)(w[q] >> 32) != tag)
                        w[q] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
#pragma unroll
            for (int q = 0; q < kCItems; ++q) {
                const int i = tid + q * kHThreads;
                if (i < D && (i < cs0 || i >= cs1) && (uint32_t)(w[q] >> 32) == tag) s_ckey[i] = __uint_as_float((uint32_t)w[q]);
            }
        }
        if (miss) s_misc[1] = 1;
        lds_barrier();
        if (s_misc[1]) {  // (uniform) score them here: keys only
            if (tid == 0 && a.status) __hip_atomic_fetch_add(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            score_items(0, D, crow, csize, s_ckey, 0, 0, 0, []() {});
            lds_barrier();
        }
    }


    // ---- 2. coarse cut under the candidate budget -----------------------
    const uint32_t cbits = block_cut<kCItems>(
        [&](int i) { return s_ckey[i]; }, [&](int i) { return s_csz[i]; }, [&](int i) { return i; }, D,
        a.cand_budget, hist, s_scan);
    // candidate flags; then the candidates in id order with their member
    // counts (prefix), and the fine candidate count F
    int nmem = 0;
#pragma unroll
    for (int j = 0; j < kCItems; ++j)
        if ((cbits >> j) & 1u) nmem += cof_r[j + 1] - cof_r[j];
    {
        // kCItems <= 32: one word of flags per thread (bits of consecutive items)
        static_assert(kCItems <= 32 && 32 % kCItems == 0, "flag packing");
        const uint32_t shifted = cbits << ((tid * kCItems) & 31);
        atomicOr(&s_cmask[(tid * kCItems) >> 5], shifted);
    }
    int2 tot2;
    const int2 ex2 = block_exclusive_sum2(make_int2(__popc(cbits), nmem), tot2, s_scan);
    const int k0 = ex2.x, ncand = tot2.x;
    int F = tot2.y;
    int m0 = ex2.y;
    // F <= candidate budget <= kHierMaxF for any state the build wrote: every
    // candidate fine cluster holds at least one of the candidates' tokens
    F = min(F, kHierMaxF);
    {
        int k = k0;
#pragma unroll
        for (int j = 0; j < kCItems; ++j) {
            if ((cbits >> j) & 1u) {
                s_ccand[k] = cof_r[j];
                s_cpre[k] = m0;
                m0 += cof_r[j + 1] - cof_r[j];
                ++k;
            }
        }
    }
    if (tid == 0) s_cpre[ncand] = F;
    if (dbg && a.dbg_candidates)
#pragma unroll
        for (int j = 0; j < kCItems; ++j) {
            const int i = tid * kCItems + j;
            if (i < D) a.dbg_candidates[(size_t)unit * D + i] = (cbits >> j) & 1u;
        }
    lds_barrier();
    for (int p = tid; p < F; p += kHThreads) {
        const int k = upper_index(s_cpre, ncand, p);
        const int f = cmem[s_ccand[k] + p - s_cpre[k]];
        s_fid[p] = f;
        s_fsz[p] = fsizes[f];
        s_foff[p] = foffs[f];  // for the exact rows, fetched with the size
    }
    lds_barrier();

    // ---- 3. fine scores of the candidates ---------------------------------
    const int fs0 = (int)((int64_t)F * rep / R), fs1 = (int)((int64_t)F * (rep + 1) / R);
    const int fsh = fs1 - fs0;  // fine share logits at s_lg[dsh .. dsh + fsh)
    // the share's first fine value rows go out now as well (row group rgi
    // takes candidates fs0 + rgi + 32 j), added after the fine cut like the
    // coarse ones: the selected among them weigh 0
    const bf16_t* fv = reinterpret_cast<const bf16_t*>(a.vbar) + (size_t)unit * a.Cmax * kHeadDim + li * 8;
    Slice8<bf16_t> pf[kHFineAhead];
    if (a.pseudo && fsh > 0) {  // (uniform)
#pragma unroll
        for (int j = 0; j < kHFineAhead; ++j)
            pf[j].load(fv + (size_t)s_fid[fs0 + min(rgi + j * kPass, fsh - 1)] * kHeadDim);
    }
    score_items(
        0, F, [&](int i) { return fk + (size_t)s_fid[i] * kHeadDim; }, [&](int i) { return s_fsz[i]; }, s_fkey, fs0,
        fs1, dsh, []() {});
    lgmax = fmaxf(lgmax, shfl_xor_f(lgmax, 16));
    lgmax = fmaxf(lgmax, shfl_xor_f(lgmax, 32));
    if (lane < G) s_gmax[wave][lane] = lgmax;
    lds_barrier();

    // reference exponent of the share's approximate terms: its largest logit
    // per head (every weight <= 1)
    SoftState<G> st;
    st.init();
    float Mref[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float m = s_gmax[0][g];
#pragma unroll
        for (int w = 1; w < kHWaves; ++w) m = fmaxf(m, s_gmax[w][g]);
        Mref[g] = m;
    }

    // ---- 4. fine cut under the token budget, in fine-id order for ties ----
    constexpr int kFItems = kHierMaxF / kHThreads;
    const uint32_t fbits = block_cut<kFItems>(
        [&](int i) { return s_fkey[i]; }, [&](int i) { return s_fsz[i]; }, [&](int i) { return s_fid[i]; }, F,
        a.budget, hist, s_scan);
    {
        static_assert(kFItems <= 32 && 32 % kFItems == 0, "flag packing");
        atomicOr(&s_fmask[(tid * kFItems) >> 5], fbits << ((tid * kFItems) & 31));
    }
    // the selected candidates in candidate order with their row prefix
    int rows_t = 0;
#pragma unroll
    for (int j = 0; j < kFItems; ++j)
        if ((fbits >> j) & 1u) rows_t += s_fsz[tid * kFItems + j];
    int2 tot4;
    const int2 ex4 = block_exclusive_sum2(make_int2(__popc(fbits), rows_t), tot4, s_scan);
    const int sk0 = ex4.x, nsel = tot4.x, E = tot4.y;
    int ro = ex4.y;
    {
        int k = sk0;
#pragma unroll
        for (int j = 0; j < kFItems; ++j) {
            const int i = tid * kFItems + j;
            if ((fbits >> j) & 1u) {
                s_sid[k] = i;
                s_spre[k] = ro;
                ro += s_fsz[i];
                ++k;
            }
        }
    }
    if (tid == 0) s_spre[nsel] = E;
    if (dbg) {
        if (a.dbg_selected) {
            __syncthreads();  // the zeros above are written
#pragma unroll
            for (int j = 0; j < kFItems; ++j)
                if ((fbits >> j) & 1u) a.dbg_selected[(size_t)unit * C + s_fid[tid * kFItems + j]] = 1;
        }
        if (tid == 0 && a.dbg_exact) a.dbg_exact[unit] = E;
    }

    // ---- 5. approximate terms of the share: coarse clusters that are not
    //      candidates, fine candidates not selected.  Weights 2^(lg - M),
    //      M the share's largest logit per head (every weight <= 1).  Row
    //      group rgi adds coarse items rgi + 32 j and fine items rgi + 32 j
    //      of the share for j below kHCoarseAhead and kHFineAhead (loaded
    //      ahead), then items rgi + 32 k of the rest, coarse before fine. ----
    if (a.pseudo) {
#pragma unroll
        for (int g = 0; g < G; ++g) st.m[g] = Mref[g];
        auto add_row = [&](const Slice8<bf16_t>& v, bool keep, int lgi) {
            float x[8];
            v.unpack(x);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float lgv = keep ? s_lg[lgi][g] : -INFINITY;
                const float w = lgv != -INFINITY ? __builtin_amdgcn_exp2f(lgv - Mref[g]) : 0.f;
                st.l[g] += w;
#pragma unroll
                for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(w, x[e], st.acc[g][e]);
            }
        };
        if (dsh > 0) {
#pragma unroll
            for (int j = 0; j < kHCoarseAhead; ++j) {
                const int t = rgi + j * kPass, c = cs0 + t;
                add_row(pv[j], t < dsh && !((s_cmask[c >> 5] >> (c & 31)) & 1u), min(t, dsh - 1));
            }
        }
        if (fsh > 0) {
#pragma unroll
            for (int j = 0; j < kHFineAhead; ++j) {
                const int i = rgi + j * kPass, fi = fs0 + i;
                add_row(pf[j], i < fsh && !((s_fmask[fi >> 5] >> (fi & 31)) & 1u), dsh + min(i, fsh - 1));
            }
        }
    }
    // the rest: coarse items [ca, dsh), then fine items [fa, fsh), as one
    // list u = 0 .. nrest - 1; lg_index(u) is the item's row of s_lg
    const int ca = min(kHCoarseAhead * kPass, dsh), fa = min(kHFineAhead * kPass, fsh);
    const int nrc = dsh - ca, nrest = nrc + fsh - fa;
    auto lg_index = [&](int u) { return u < nrc ? ca + u : dsh + fa + (u - nrc); };
    for (int u = tid; u < nrest; u += kHThreads) {
        const int t = lg_index(u);
        bool keep;
        if (t < dsh) {
            const int c = cs0 + t;
            keep = !((s_cmask[c >> 5] >> (c & 31)) & 1u);
        } else {
            const int i = fs0 + t - dsh;
            keep = !((s_fmask[i >> 5] >> (i & 31)) & 1u);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float lgv = s_lg[t][g];
            s_lg[t][g] = keep && lgv != -INFINITY ? __builtin_amdgcn_exp2f(lgv - Mref[g]) : 0.f;
        }
    }
    if (a.pseudo && nrest > 0) {  // (uniform)
        lds_barrier();
        auto vrow = [&](int u) {
            const int t = lg_index(u);
            return t < dsh ? cv + (size_t)(cs0 + t) * kHeadDim : fv + (size_t)s_fid[fs0 + t - dsh] * kHeadDim;
        };
        // 32 row groups, one row each per pass, two passes in flight
        Slice8<bf16_t> v[2];
        v[0].load(vrow(rgi < nrest ? rgi : 0));
        v[1].load(vrow(rgi + kPass < nrest ? rgi + kPass : 0));
        auto absorb = [&](const Slice8<bf16_t>& vr, int u) {
            float x[8];
            vr.unpack(x);
            const int t = lg_index(u < nrest ? u : 0);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float w = u < nrest ? s_lg[t][g] : 0.f;
                st.l[g] += w;
#pragma unroll
                for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(w, x[e], st.acc[g][e]);
            }
        };
        // the last two passes are taken without loading rows past the end
        int u0 = 0;
        for (; u0 + 2 * kPass < nrest; u0 += 2 * kPass) {
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int u = u0 + k * kPass + rgi;
                absorb(v[k], u);
                const int un = u + 2 * kPass;
                v[k].load(vrow(un < nrest ? un : 0));
            }
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) absorb(v[k], u0 + k * kPass + rgi);
    }

    // ---- 6. exact rows of the share: selected members [0, E), then the
    //      unclustered tail [E, E + Tn) (staged as -1 - token, read from K, V)
    const float qscale = kInvSqrtD * kLog2e;
    const size_t ubase = (size_t)unit * a.Nmax * kHeadDim;
    const int32_t* tids = a.token_ids ? a.token_ids + (size_t)unit * a.Nmax : nullptr;
    const int Tn = a.n_total - a.n_clustered;
    const int Et = E + Tn;
    const int e0 = (int)((int64_t)Et * rep / R), e1 = (int)((int64_t)Et * (rep + 1) / R);
    {
        const bf16_t* Kx = reinterpret_cast<const bf16_t*>(a.Kx) + ubase;
        const bf16_t* Vx = reinterpret_cast<const bf16_t*>(a.Vx) + ubase + li * 8;
        const bf16_t* Kt = reinterpret_cast<const bf16_t*>(a.K) + ubase;
        const bf16_t* Vt = reinterpret_cast<const bf16_t*>(a.V) + ubase + li * 8;
        float mv = exact16_enter<G>(st);
        float lp = 0.f;
        float* sp = s_p + wave * 16 * G;
        for (int c0 = e0; c0 < e1; c0 += kHRowBatch) {
            const int cnt = min(kHRowBatch, e1 - c0);
            lds_barrier();  // the previous batch is consumed
            for (int i = tid; i < cnt; i += kHThreads) {
                const int r = c0 + i;
                int v;
                if (r < E) {  // member r - pre[k] of selected candidate k
                    const int k = upper_index(s_spre, nsel, r);
                    const int pos = s_foff[s_sid[k]] + r - s_spre[k];
                    v = tids ? tids[pos] : pos;
                } else {
                    v = -1 - (a.n_clustered + r - E);
                }
                s_row[i] = v;
            }
            lds_barrier();
            const int nb = (cnt + 15) / 16;
            auto blk = [&](int step) {
                const int q = step * kHWaves + wave;
                return q < nb ? q : nb;  // nb: past the end, masked
            };
            auto load_step = [&](ExactRows16& rr, int step) {
                const int ib = blk(step) * 16;
                const int ik = ib + li;
                const int rk = s_row[ik < cnt ? ik : 0];
                load_row_blocks(rr.k, rk >= 0 ? Kx + (size_t)rk * kHeadDim : Kt + (size_t)(-1 - rk) * kHeadDim, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int iv = ib + 4 * rg + e;
                    const int rv = s_row[iv < cnt ? iv : 0];
                    rr.v[e].load(rv >= 0 ? Vx + (size_t)rv * kHeadDim : Vt + (size_t)(-1 - rv) * kHeadDim);
                }
            };
            ExactRows16 ring[kHExactDepth];
#pragma unroll
            for (int j = 0; j < kHExactDepth; ++j) {
                load_step(ring[j], j);
                __builtin_amdgcn_sched_barrier(0);
            }
            const int steps = (nb + kHWaves - 1) / kHWaves;
            // the last group is consumed without loading further rows
            int it = 0;
            for (; it + kHExactDepth < steps; it += kHExactDepth) {
#pragma unroll
                for (int j = 0; j < kHExactDepth; ++j) {
                    exact16_step<G>(st, mv, lp, sp, qop, ring[j], blk(it + j) * 16 + 4 * rg, cnt, qscale);
                    load_step(ring[j], it + j + kHExactDepth);
                    __builtin_amdgcn_sched_barrier(0);
                }
            }
#pragma unroll
            for (int j = 0; j < kHExactDepth; ++j)
                exact16_step<G>(st, mv, lp, sp, qop, ring[j], blk(it + j) * 16 + 4 * rg, cnt, qscale);
        }
        exact16_leave<G>(st, mv, lp);
    }

    // ---- 7. combine the workgroup's states; the last workgroup of the unit
    //      merges the partials and writes the output -------------------------
    finish_step<G, kHWaves>(st, s_red, s_misc, a.out + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim,
                            a.xpart + (size_t)unit * R * G * (kHeadDim + 2), a.xcount + unit, tag, a.xepoch + unit,
                            a.status, R, rep, kHPartialWaitTicks);
}

// Workgroups per unit: enough for about 256 workgroups in all (one per
// compute unit), at least 3.  Every phase reads a few tens of KB per
// workgroup and a compute unit streams some 30 GB/s, so smaller shares
// shorten each phase more than the extra partners lengthen the key exchange
// (8 per unit at 32 units measured 1 us faster than 4).
int hier_replicas(int units) {
    constexpr int kWorkgroups = 256;
    int r = kHierMinReplicas;
    while (units * r < kWorkgroups && r < kHierMaxReplicas) ++r;
    return r;
}

bool hier_path_fits(int dtype, int G, int max_coarse, int cand_budget) {
    return dtype == 1 && (G == 1 || G == 2 || G == 4) && max_coarse >= 1 && max_coarse <= kHierMaxD &&
           cand_budget >= 0 && cand_budget <= kHierMaxF;
}

hipError_t launch_hier_decode(int dtype, int G, const HierArgs& a, int units, int replicas, hipStream_t st) {
    if (!hier_path_fits(dtype, G, a.D, a.cand_budget) || a.D > a.Dmax || replicas < kHierMinReplicas ||
        replicas > kHierMaxReplicas || !a.out || !a.xch || !a.xpart || !a.xcount || !a.xepoch)
        return hipErrorInvalidValue;
    dim3 grid(units, replicas);
    switch (G) {
        case 1: hipLaunchKernelGGL(hier_decode_kernel<1>, grid, dim3(kHThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(hier_decode_kernel<2>, grid, dim3(kHThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL(hier_decode_kernel<4>, grid, dim3(kHThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mpa
