// unit.hip -- one Multipole Attention decode step of a (sequence, KV head)
// unit in one launch: R workgroups of 512 threads per unit (R = 1 when the
// batch has 256 units or more and at most 2048 clusters per unit).
//
// Pages: atlas.scime.ai summary, opening sentence (exact attention on the
// top-scoring clusters, centroid attention for the rest) and "Approach"
// (value centroids stand in for the unselected clusters); mlsanity.com paper
// page, "Abstract (arXiv)" (centroids pick the important keys).
//
// Workgroup r of a unit:
//   1. scores its share [C r / R, C (r + 1) / R) of the clusters on the
//      matrix cores and takes the other shares' ranking keys from the other
//      workgroups as tagged 64-bit words (or scores them itself when a
//      partner is late: the same bits);
//   2. splits its waves: waves 0-3 take the budget cut (a size-weighted LDS
//      histogram over value bins, radix passes when that does not settle
//      it) while waves 4-7 stream the approximate term n exp(s) Vbar of
//      every cluster of the share; the selected clusters' terms are taken
//      back out afterwards;
//   3. attends its share of the exact rows (the selected clusters' members,
//      then the unclustered tail) on the matrix cores;
//   4. combines its waves; the last workgroup of the unit to finish merges the
//      partials and writes the output (finish_step).
// No score, cut record or selection list leaves the workgroup, and there is
// no launch boundary between the steps.  The split launches in decode.hip
// serve the configurations this path does not take.
#include <math.h>

#include <type_traits>

#include "attn.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

constexpr int kUnitThreads = 512;
constexpr int kUnitWaves = kUnitThreads / kWave;  // 8
constexpr int kUnitRowBatch = 1024;               // staged exact rows per pass
// Three shapes: up to 2048 clusters with one replica per unit (the whole
// approximate term in one workgroup), up to 2048 or 4096 clusters with
// shares of up to 1024 per replica.
constexpr int kUnitMaxCSmall = 2048, kUnitShareSmall = 2048;
constexpr int kUnitMaxCLarge = 4096, kUnitShareLarge = 1024;

// Barrier of waves 0 .. NW-1 of the workgroup through an LDS counter, the
// other waves running on.  Each of those waves passes the same sequence of
// these barriers (gen counts them), and all of them are resident, so the
// wait always ends.
template <int NW>
__device__ __forceinline__ void group_barrier(int* ctr, int& gen) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    ++gen;
    if ((threadIdx.x & (kWave - 1)) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    while (__hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < NW * gen) __builtin_amdgcn_s_sleep(1);
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Number of threads of waves 0 .. NW-1 with p set (`lds`: NW ints, free
// again after the next group barrier).
template <int NW>
__device__ __forceinline__ int group_count(bool p, int* lds, int* ctr, int& gen) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int c = __popcll(__ballot(p));
    if (lane == 0) lds[wave] = c;
    group_barrier<NW>(ctr, gen);
    int t = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) t += lds[w];
    return t;
}

// Exclusive scan of two counters over waves 0 .. NW-1 in thread order;
// totals in tot (`lds`: 2 NW ints).
template <int NW>
__device__ __forceinline__ int2 group_exclusive_sum2(int2 v, int2& tot, int* lds, int* ctr, int& gen) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
    const int ix = wave_inclusive_sum(v.x), iy = wave_inclusive_sum(v.y);
    if (lane == kWave - 1) {
        lds[2 * wave] = ix;
        lds[2 * wave + 1] = iy;
    }
    group_barrier<NW>(ctr, gen);
    int bx = 0, by = 0, tx = 0, ty = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const int p = lds[2 * w], q = lds[2 * w + 1];
        if (w < wave) {
            bx += p;
            by += q;
        }
        tx += p;
        ty += q;
    }
    group_barrier<NW>(ctr, gen);  // lds may be reused right after
    tot = make_int2(tx, ty);
    return make_int2(bx + ix - v.x, by + iy - v.y);
}

// Budget cut taken by waves 0 .. NW-1 (the others run on): the longest prefix
// of the non-empty clusters in (key desc, id asc) order whose sizes sum to at
// most `budget`.  Thread t owns clusters ITEMS t .. ITEMS t + ITEMS - 1.  A
// pass over equal-width value bins (range_cut) usually settles it.  Else four
// 8-bit radix passes over the order-preserving key bits of the clusters still
// open, weighted by size, into LDS histograms find the cut value (every wave
// scans the histogram and reaches the same digit); clusters above it are
// selected, clusters equal to it in id order while they fit.  One group scan
// places the selected clusters in id order: ids, first members, member-row
// prefix (s_spre[nsel] = E), and nsel, E in out[0], out[1]; marks[0] and
// marks[1] receive the number of selected clusters with an id below mark_lo
// and mark_hi.
template <int NW, int ITEMS>
__device__ __forceinline__ void group_cut(const float* s_key, const int32_t* s_sz, const int32_t* s_off,
                                          const int32_t* s_rows, int C, int budget, int (*hist)[256], int* s_scan,
                                          int* ctr, int& gen, int32_t* s_sid, int32_t* s_soff, int32_t* s_spre,
                                          int* out, int32_t* dbg_sel, int mark_lo, int mark_hi, int* marks) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    uint32_t key[ITEMS];
    float kf[ITEMS];
    int isz[ITEMS];
    uint32_t act = 0, selbits = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = tid * ITEMS + j;
        kf[j] = i < C ? s_key[i] : 0.f;
        key[j] = order_key(kf[j]);
        isz[j] = i < C ? s_sz[i] : 0;
        act |= (uint32_t)(isz[j] > 0) << j;
    }
    int Rb = budget;
    auto bar = [&]() { group_barrier<NW>(ctr, gen); };
    if (!range_cut<NW, ITEMS>(kf, key, isz, [&](int j) { return tid * ITEMS + j; }, Rb, act, selbits,
                              reinterpret_cast<unsigned long long*>(&hist[0][0]), reinterpret_cast<float*>(s_scan),
                              bar)) {  // (uniform, rare) exact radix passes over the open items
        int rsz[ITEMS];
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) rsz[j] = ((act >> j) & 1u) ? isz[j] : 0;
        bar();  // the first pass's histogram is read
        for (int k = tid; k < 4 * 256; k += NW * kWave) reinterpret_cast<int*>(hist)[k] = 0;
        bar();
        uint32_t prefix = 0, pmask = 0;
        bool done = false;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            const int shift = 24 - 8 * p;
#pragma unroll
            for (int j = 0; j < ITEMS; ++j)
                if (rsz[j] > 0 && (key[j] & pmask) == prefix) atomicAdd(&hist[p][(key[j] >> shift) & 255u], rsz[j]);
            bar();
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
        int tie_local = 0;
        if (!done) {
#pragma unroll
            for (int j = 0; j < ITEMS; ++j)
                if (rsz[j] > 0 && key[j] == prefix) tie_local += rsz[j];
        }
        int run_tie = 0;
        if (!done && group_count<NW>(tie_local > 0, s_scan + 32, ctr, gen) > 1) {  // uniform
            int2 tt;
            run_tie = group_exclusive_sum2<NW>(make_int2(tie_local, 0), tt, s_scan, ctr, gen).x;
        }
#pragma unroll
        for (int j = 0; j < ITEMS; ++j) {
            bool sel;
            if (done) {
                sel = key[j] >= prefix;  // prefix: the digits fixed so far, low bits zero
            } else {
                const bool tie = key[j] == prefix;
                sel = key[j] > prefix || (tie && run_tie + rsz[j] <= Rb);
                if (tie) run_tie += rsz[j];
            }
            selbits |= (uint32_t)(sel && rsz[j] > 0) << j;
        }
    }
    int s_local = 0, rows_local = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const bool sel = (selbits >> j) & 1u;
        s_local += sel;
        rows_local += sel ? s_rows[tid * ITEMS + j] : 0;
    }
    int2 tot;
    const int2 ex = group_exclusive_sum2<NW>(make_int2(s_local, rows_local), tot, s_scan, ctr, gen);
    int k = ex.x, ro = ex.y;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        const int i = tid * ITEMS + j;
        if (i == mark_lo) marks[0] = k;
        if (i == mark_hi) marks[1] = k;
        if ((selbits >> j) & 1u) {
            s_sid[k] = i;
            s_soff[k] = s_off[i];
            s_spre[k] = ro;
            ++k;
            ro += s_rows[i];
        }
        if (dbg_sel && i < C) dbg_sel[i] = (selbits >> j) & 1u;
    }
    if (tid == 0) {
        s_spre[tot.x] = tot.y;
        out[0] = tot.x;
        out[1] = tot.y;
        if (mark_hi >= NW * kWave * ITEMS) marks[1] = tot.x;
    }
}

// LDS layout (bytes).  The final reduction of the waves' states reuses the
// "big" region once the selection lists, weights and row stage are dead.
template <int G, int kUnitMaxC, int kUnitShare>
struct UnitLds {
    static constexpr int key = 0;                                    // float [MaxC]
    static constexpr int sz = key + kUnitMaxC * 4;                   // int [MaxC]: sizes
    static constexpr int off = sz + kUnitMaxC * 4;                   // int [MaxC]: first member
    static constexpr int rows = off + kUnitMaxC * 4;                 // int [MaxC]: member rows
    static constexpr int hist = rows + kUnitMaxC * 4;                // int [4][256]
    static constexpr int scan = hist + 4 * 256 * 4;                  // int [64]
    static constexpr int misc = scan + 64 * 4;                       // int [8]
    static constexpr int gmax = misc + 8 * 4;                        // float [waves][G]
    static constexpr int pexp = gmax + kUnitWaves * G * 4;          // float [waves][16][G]
    static constexpr int big = pexp + kUnitWaves * 16 * G * 4;
    static constexpr int sid = big;                                  // int [MaxC]
    static constexpr int soff = sid + kUnitMaxC * 4;                 // int [MaxC]
    static constexpr int spre = soff + kUnitMaxC * 4;                // int [MaxC + 1]
    static constexpr int lg = spre + (kUnitMaxC + 4) * 4;            // float [Share][G]
    static constexpr int row = lg + kUnitShare * G * 4;              // int [RowBatch]
    static constexpr int big_end = row + kUnitRowBatch * 4;
    static constexpr int red_bytes = kUnitWaves * G * (kHeadDim + 2) * 4;
    static constexpr int bytes = (big_end > big + red_bytes ? big_end : big + red_bytes);
    static_assert(hist % 16 == 0 && 256 * 8 + kRankCap * 16 <= 4 * 256 * 4, "value-bin pass in the histogram");
};

constexpr int kScoreDepth = 4;                           // score steps in flight per wave
constexpr int kPseudoDepth = 2;                          // value-centroid steps in flight per wave
constexpr int kExactDepth = 2;                           // exact-row steps (16 rows) in flight per wave
// sixteenths of the first batch of exact rows that waves 0-3 take (they
// start on it while waves 4-7 finish the approximate term)
constexpr int kFirstBatchEarly = 11;
// Waits on the other replicas of a unit, in ticks of the 100 MHz constant
// clock: for their keys (then the workgroup scores them itself) and for the
// partial words of replicas that have already counted in.
constexpr uint64_t kExchangeWaitTicks = 2000;
constexpr uint64_t kPartialWaitTicks = 100000;

// Four rows of a row group (one ring step of the score or the value-centroid
// stream).
template <typename T>
struct Rows4 {
    Slice8<T> r[4];
};

// F8: the centroids come from their fp8 copies (codes and scale bytes).
template <typename T, int G, int kUnitMaxC, int kUnitShare, bool F8>
__global__ __launch_bounds__(kUnitThreads) void unit_decode_kernel(UnitArgs a) {
    constexpr int kUnitRecItems = kUnitMaxC / kUnitThreads;        // cluster records per thread
    using L = UnitLds<G, kUnitMaxC, kUnitShare>;
    __shared__ __align__(16) char lds[L::bytes];
    float* s_key = reinterpret_cast<float*>(lds + L::key);
    int32_t* s_sz = reinterpret_cast<int32_t*>(lds + L::sz);
    int32_t* s_off = reinterpret_cast<int32_t*>(lds + L::off);
    int32_t* s_rows = reinterpret_cast<int32_t*>(lds + L::rows);
    int(*hist)[256] = reinterpret_cast<int(*)[256]>(lds + L::hist);
    int* s_scan = reinterpret_cast<int*>(lds + L::scan);
    int* s_misc = reinterpret_cast<int*>(lds + L::misc);
    float(*s_gmax)[G] = reinterpret_cast<float(*)[G]>(lds + L::gmax);
    float* s_p = reinterpret_cast<float*>(lds + L::pexp);
    int32_t* s_sid = reinterpret_cast<int32_t*>(lds + L::sid);
    int32_t* s_soff = reinterpret_cast<int32_t*>(lds + L::soff);
    int32_t* s_spre = reinterpret_cast<int32_t*>(lds + L::spre);
    float(*s_lg)[G] = reinterpret_cast<float(*)[G]>(lds + L::lg);
    int32_t* s_row = reinterpret_cast<int32_t*>(lds + L::row);
    float(*s_red)[G][kHeadDim + 2] = reinterpret_cast<float(*)[G][kHeadDim + 2]>(lds + L::big);

    // grid (unit, replica): the replicas of a unit are U workgroups apart in
    // dispatch order, so with U a multiple of 8 they land on the same XCD and
    // share its L2 for the key centroids both of them read
    const int unit = blockIdx.x, rep = blockIdx.y, R = gridDim.y;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int C = a.C;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    // the call's tag of the unit's exchange words: one more than the tag of
    // its last decode (0 is never a tag: a zeroed word matches no call)
    uint32_t tag = 0;
    if (R > 1) {
        tag = a.xepoch[unit] + 1u;
        if (tag == 0u) tag = 1u;
    }
    const int su = unit / a.ugroup;  // the unit's clusters and cache (shared by a group when per head)
    const int32_t* szu = a.sizes + (size_t)su * a.Cmax;
    const int32_t* ofu = a.offsets + (size_t)su * (a.Cmax + 1);
    const int cs = (int)((int64_t)C * rep / R), ce = (int)((int64_t)C * (rep + 1) / R);  // approximate-term share

    const bf16_t* qg = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim;
    const bf16_t* cu = reinterpret_cast<const bf16_t*>(a.kbar) + (size_t)su * a.Cmax * kHeadDim;
    constexpr int kScaleBytes = kHeadDim / 32;  // fp8 copies: one scale byte per 32 values
    const uint8_t* kc = F8 ? a.kcodes + (size_t)su * a.Cmax * kHeadDim : nullptr;
    const uint8_t* ksc = F8 ? a.kscales + (size_t)su * a.Cmax * kScaleBytes : nullptr;
    // one key-centroid row of the score ring: the lane's 4 operand blocks, or
    // its 32 codes and their scale
    using KRow = std::conditional_t<F8, KCodes, Rows4<bf16_t>>;
    auto kload = [&](KRow& r, int i) {
        if constexpr (F8)
            r.load(kc + (size_t)i * kHeadDim, ksc + (size_t)i * kScaleBytes, rg);
        else
            load_row_blocks(r.r, cu + (size_t)i * kHeadDim, lane);
    };
    // one pass over clusters [lo, hi) by nw waves (this one is wave wv of
    // them); the first pass (all waves) also brings the cluster records to
    // LDS while its first centroid rows are in flight, and only it writes the
    // share's logits (the approximate term may have replaced them with its
    // weights by the time a later pass runs)
    float lgmax = -INFINITY;  // the lane's maximum share logit (head li)
    auto score_pass = [&](int lo, int hi, bool first, int nw, int wv) {
        // the cluster records (first pass) go out ahead of the centroid rows,
        // as unconditional loads (clamped index), so writing them to LDS waits
        // for them alone and not for the ring behind them
        int rsz[kUnitRecItems], ro0[kUnitRecItems], ro1[kUnitRecItems];
        if (first) {
#pragma unroll
            for (int j = 0; j < kUnitRecItems; ++j) {
                const int i = min(tid + j * kUnitThreads, C - 1);
                rsz[j] = szu[i];
                ro0[j] = ofu[i];
                ro1[j] = ofu[i + 1];
            }
        }
        QOperand qop;
        if constexpr (F8)
            load_qop_blocks<G>(qop, qg, lane);
        else
            load_qop<G>(qop, qg, lane);
        // the waves interleave: one step of the workgroup reads 16 nw
        // consecutive clusters, so the workgroup is a single stream; lane l
        // loads row l % 16 of its wave's 16
        const int steps = (hi - lo + 16 * nw - 1) / (16 * nw);
        auto base = [&](int step) { return lo + step * 16 * nw + wv * 16; };
        KRow ring[kScoreDepth];
#pragma unroll
        for (int j = 0; j < kScoreDepth; ++j) {
            const int i = base(j) + li;
            kload(ring[j], i < hi ? i : max(hi - 1, 0));
            __builtin_amdgcn_sched_barrier(0);
        }
        if (first) {
#pragma unroll
            for (int j = 0; j < kUnitRecItems; ++j) {
                const int i = tid + j * kUnitThreads;
                if (i < C) {
                    s_sz[i] = rsz[j];
                    s_off[i] = ro0[j];
                    s_rows[i] = ro1[j] - ro0[j];
                }
            }
            for (int k = tid; k < 4 * 256; k += kUnitThreads) reinterpret_cast<int*>(hist)[k] = 0;
            lds_barrier();
        }
        // step s from ring slot r: lane (rg, li) receives rows 4 rg + e of
        // the 16 for head li; rows past the end store nothing
        auto consume = [&](const KRow& r, int s) {
            f32x4v d;
            if constexpr (F8) {
                Slice8<bf16_t> op[4];
                r.operands(op);
                d = mfma_scores(op, qop);
            } else {
                d = mfma_scores(r.r, qop);
            }
            const int cb = base(s) + 4 * rg;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float sv = d[e] * kInvSqrtD;
                const float key = head_mean<G>(sv);
                const int i = cb + e;
                if (i < hi) {
                    if (li == 0) s_key[i] = key;
                    if (li < G) {
                        if (a.dbg_scores) a.dbg_scores[((size_t)unit * C + i) * G + li] = sv;
                        if (first && i >= cs && i < ce) {  // later passes keep them
                            const int n = s_sz[i];
                            const float lgv = n > 0 ? fmaf(sv, kLog2e, log2_count(n)) : -INFINITY;
                            s_lg[i - cs][li] = lgv;
                            lgmax = fmaxf(lgmax, lgv);
                        }
                    }
                }
            }
        };
        // the ring's last group is consumed without loading further rows, so
        // nothing is left in flight when the pass ends (a later wait would
        // include it); rows past the end of a partial step read the range's
        // last row, or row 0 when the range is empty (fewer clusters than
        // replicas): a cached row
        int it = 0;
        for (; it + kScoreDepth < steps; it += kScoreDepth) {
#pragma unroll
            for (int j = 0; j < kScoreDepth; ++j) {
                consume(ring[j], it + j);
                const int i = base(it + j + kScoreDepth) + li;
                kload(ring[j], i < hi ? i : max(hi - 1, 0));
                __builtin_amdgcn_sched_barrier(0);  // keep the ring order
            }
        }
#pragma unroll
        for (int j = 0; j < kScoreDepth; ++j) consume(ring[j], it + j);
        if (first) {  // the wave's maximum logit of head li over the share
            lgmax = fmaxf(lgmax, shfl_xor_f(lgmax, 16));
            lgmax = fmaxf(lgmax, shfl_xor_f(lgmax, 32));
            if (lane < G) s_gmax[wave][lane] = lgmax;
        }
    };

    // ---- scores on the matrix cores through a ring of kScoreDepth steps:
    //      step s of wave w takes clusters lo + 128 s + 16 w .. + 16.  The
    //      ranking key goes to LDS, the share's base-2 logits s log2(e) +
    //      log2(n) too.  The ring body has no data-dependent branch (steps
    //      past the end load row 0 and store nothing), so the compiler's wait
    //      counts stay exact.  With several replicas each scores only its
    //      share and the keys of the others come through the exchange below.
    score_pass(R > 1 ? cs : 0, R > 1 ? ce : C, true, kUnitWaves, wave);
    lds_barrier();

    // ---- approximate terms of the share: the value centroids of clusters
    //      [cs, ce), weighted by 2^(lg - M) with M the share's maximum logit
    //      over all its clusters (from the score pass; every weight is at most
    //      1), stream through a ring of kPseudoDepth steps of 4 rows per row
    //      group.  Waves 4-7 run it over every cluster of the share while
    //      waves 0-3 take the cut; the selected clusters are taken out after.
    const T* vb = reinterpret_cast<const T*>(a.vbar) + (size_t)su * a.Cmax * kHeadDim + li * 8;
    const uint8_t* vc = F8 ? a.vcodes + (size_t)su * a.Cmax * kHeadDim + li * 8 : nullptr;
    const uint8_t* vsc = F8 ? a.vscales + (size_t)su * a.Cmax * kScaleBytes + (li >> 2) : nullptr;
    // values li * 8 .. + 7 of value-centroid row c
    using VRow = std::conditional_t<F8, VCodes8, Slice8<T>>;
    auto vload = [&](VRow& v, int c) {
        if constexpr (F8)
            v.load(vc + (size_t)c * kHeadDim, vsc + (size_t)c * kScaleBytes);
        else
            v.load(vb + (size_t)c * kHeadDim);
    };
    constexpr int kCutWaves = 4, kStreamWaves = kUnitWaves - kCutWaves;
    constexpr int kSteps = kUnitShare / (16 * kStreamWaves);
    // every step of the stream lies inside the share
    static_assert(kUnitShare % (16 * kStreamWaves) == 0 && kSteps % kPseudoDepth == 0, "stream steps");
    const int sw = wave - kCutWaves;  // stream wave index (waves 4-7)
    auto item = [&](int step, int u) { return step * 16 * kStreamWaves + sw * 16 + u * 4 + rg; };
    struct VRows4 {
        VRow r[4];
    };
    VRows4 pring[kPseudoDepth];
    SoftState<G> st;
    st.init();
    // the first batch of the removal (below): rows in flight through the exact
    // rows, weights relative to Mref (0: no row), applied after them
    constexpr int kRemoveBatch = 4;
    VRow rem_v[kRemoveBatch];
    float rem_p[kRemoveBatch][G];
#pragma unroll
    for (int j = 0; j < kRemoveBatch; ++j)
#pragma unroll
        for (int g = 0; g < G; ++g) rem_p[j][g] = 0.f;
    float Mref[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float m = s_gmax[0][g];
#pragma unroll
        for (int w = 1; w < kUnitWaves; ++w) m = fmaxf(m, s_gmax[w][g]);
        Mref[g] = m;
    }

    // ---- key exchange between the replicas of the unit.  Every replica
    //      writes the keys of its share into each other replica's slot as
    //      64-bit words (call tag << 32 | key bits) with agent-scope atomic
    //      stores; waves 0-3 then read its own slot: a word counts once it
    //      carries this call's tag, so no fence or flag orders the words, and
    //      words of earlier calls (other tags) need no clearing.  A word still
    //      missing after kExchangeWaitTicks (a replica not yet running) makes
    //      waves 0-3 score every cluster themselves with the same operations,
    //      which gives the same keys. ------------------------------------------
    const uint64_t tagw = (uint64_t)tag << 32;
    uint64_t* xu = a.xch + (size_t)unit * R * a.Cmax;
    if (R > 1 && !a.rescore) {
        for (int i = cs + tid; i < ce; i += kUnitThreads) {
            const uint64_t w = tagw | __float_as_uint(s_key[i]);
            for (int r2 = 0; r2 < R; ++r2)
                if (r2 != rep)
                    __hip_atomic_store(xu + (size_t)r2 * a.Cmax + i, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (a.pseudo) {
#pragma unroll
        for (int g = 0; g < G; ++g) st.m[g] = Mref[g];
    }
    if (R > 1 && a.rescore == 1) {  // every wave scores the other shares too
        score_pass(0, C, false, kUnitWaves, wave);
    }
    int* gctr = s_misc + 5;  // group barrier counters: waves 0-3, waves 4-7
    int* sctr = s_misc + 4;
    int* rflag = s_misc + 3;  // set once waves 0-3 have staged the first batch of exact rows
    if (tid == 0) {
        *gctr = 0;
        *sctr = 0;
        *rflag = 0;
    }
    lds_barrier();
    // exact rows of the replica: the selected clusters' members [0, E), then
    // the unclustered tail [E, E + Tn); this replica takes [e0, e1) of them,
    // in batches of kUnitRowBatch staged in s_row (a member position, or -1 -
    // token for a tail row, read from K, V)
    const int Tn = a.n_total - a.n_clustered;
    const int32_t* tids = a.token_ids ? a.token_ids + (size_t)su * a.Nmax : nullptr;
    // threads t0, t0 + nt, ... take the selected clusters in turn and write
    // the positions of their members that fall in the batch (no search: a
    // cluster's rows are [pre[k], pre[k + 1]) at first member off[k]), then
    // the tail rows of the batch
    auto stage = [&](int c0, int cnt, int nsel, int E, int t0, int nt) {
        const int c1 = c0 + cnt;
        for (int k = t0; k < nsel; k += nt) {
            const int p0 = s_spre[k], p1 = s_spre[k + 1];
            const int lo = max(p0, c0), hi = min(p1, c1);
            const int off = s_soff[k] - p0;
            if (tids) {
                for (int r = lo; r < hi; ++r) s_row[r - c0] = tids[off + r];
            } else {
                for (int r = lo; r < hi; ++r) s_row[r - c0] = off + r;
            }
        }
        for (int i = max(E - c0, 0) + t0; i < cnt; i += nt) s_row[i] = -1 - (a.n_clustered + c0 + i - E);
    };
    auto row_range = [&](int E, int& e0, int& e1) {
        const int Et = E + Tn;
        e0 = (int)((int64_t)Et * rep / R);
        e1 = (int)((int64_t)Et * (rep + 1) / R);
    };

    if (wave < kCutWaves) {
        // ---- waves 0-3: the other replicas' keys, then the budget cut -------
        int gen = 0;
        if (R > 1 && a.rescore != 1) {
            bool miss = a.rescore == 2;  // 2: as if the other keys never came
            if (!miss) {
                constexpr int kPoll = kUnitMaxC / (kCutWaves * kWave);  // words per thread
                uint64_t* slot = xu + (size_t)rep * a.Cmax;
                uint64_t w[kPoll];
#pragma unroll
                for (int q = 0; q < kPoll; ++q)  // unconditional (clamped): exact wait counts
                    w[q] = __hip_atomic_load(slot + min(tid + q * kCutWaves * kWave, C - 1), __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
                bool fresh = true;
#pragma unroll
                for (int q = 0; q < kPoll; ++q) {
                    const int i = tid + q * kCutWaves * kWave;
                    fresh = fresh && (!(i < C && (i < cs || i >= ce)) || (uint32_t)(w[q] >> 32) == tag);
                }
                if (!fresh) {  // a partner is behind: poll its words, for a bounded time
                    // every stale word of the thread is read again in one
                    // batch per round, so a round costs one trip to L2
                    const uint64_t t0 = wall_clock64();
                    for (;;) {
                        bool stale = false;
#pragma unroll
                        for (int q = 0; q < kPoll; ++q) {
                            const int i = tid + q * kCutWaves * kWave;
                            stale = stale || (i < C && (i < cs || i >= ce) && (uint32_t)(w[q] >> 32) != tag);
                        }
                        if (!stale) break;
                        if (wall_clock64() - t0 > kExchangeWaitTicks) {
                            miss = true;
                            break;
                        }
                        __builtin_amdgcn_s_sleep(2);
#pragma unroll
                        for (int q = 0; q < kPoll; ++q) {
                            const int i = tid + q * kCutWaves * kWave;
                            if (i < C && (i < cs || i >= ce) && (uint32_t)(w[q] >> 32) != tag)
                                w[q] = __hip_atomic_load(slot + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
#pragma unroll
                for (int q = 0; q < kPoll; ++q) {
                    const int i = tid + q * kCutWaves * kWave;
                    if (i < C && (i < cs || i >= ce) && (uint32_t)(w[q] >> 32) == tag)
                        s_key[i] = __uint_as_float((uint32_t)w[q]);
                }
            }
            if (group_count<kCutWaves>(miss, s_scan + 32, gctr, gen) > 0) {
                if (tid == 0 && a.status)
                    __hip_atomic_fetch_add(a.status, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                score_pass(0, C, false, kCutWaves, wave);  // these four waves
            }
            group_barrier<kCutWaves>(gctr, gen);
        }
        group_cut<kCutWaves, kUnitMaxC / (kCutWaves * kWave)>(
            s_key, s_sz, s_off, s_rows, C, a.budget, hist, s_scan, gctr, gen, s_sid, s_soff, s_spre, s_misc + 6,
            a.dbg_selected && rep == 0 ? a.dbg_selected + (size_t)unit * C : nullptr, cs, ce, s_misc + 1);
        group_barrier<kCutWaves>(gctr, gen);  // the whole list is written
        {
            // the first batch of exact rows, staged while waves 4-7 still
            // stream the approximate term; the flag lets them in after it
            int e0, e1;
            row_range(s_misc[7], e0, e1);
            stage(e0, min(kUnitRowBatch, e1 - e0), s_misc[6], s_misc[7], tid, kCutWaves * kWave);
            group_barrier<kCutWaves>(gctr, gen);
            if (tid == 0) __hip_atomic_store(rflag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (a.pseudo) {
            // take the selected clusters of the share [cs, ce) (a contiguous
            // run of the ascending selected list) back out of the approximate
            // term, with the weights waves 4-7 computed (their first barrier)
            while (__hip_atomic_load(sctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < kStreamWaves)
                __builtin_amdgcn_s_sleep(1);
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
            // the share's run of the selected list, counted by the cut
            const int k_lo = s_misc[1], k_hi = s_misc[2];
            // 16 row groups take kRemoveBatch rows each per pass, the loads
            // of a pass in flight together.  The first pass is only issued
            // here: its rows are taken out after the exact rows, so their
            // latency hides behind them; further passes (more than 64
            // selected clusters in the share) run now.
            const int rgi = wave * 4 + rg;
#pragma unroll
            for (int j = 0; j < kRemoveBatch; ++j) {
                const int k = k_lo + 16 * j + rgi;
                const int c = k < k_hi ? s_sid[k] : -1;
                vload(rem_v[j], c >= 0 ? c : cs);
#pragma unroll
                for (int g = 0; g < G; ++g) rem_p[j][g] = c >= 0 ? s_lg[c - cs][g] : 0.f;
            }
            for (int k0 = k_lo + 16 * kRemoveBatch; k0 < k_hi; k0 += 16 * kRemoveBatch) {
                VRow v[kRemoveBatch];
                int c[kRemoveBatch];
#pragma unroll
                for (int j = 0; j < kRemoveBatch; ++j) {
                    const int k = k0 + 16 * j + rgi;
                    c[j] = k < k_hi ? s_sid[k] : -1;
                    vload(v[j], c[j] >= 0 ? c[j] : cs);
                }
#pragma unroll
                for (int j = 0; j < kRemoveBatch; ++j) {
                    float x[8];
                    v[j].unpack(x);
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        // every state's reference is still Mref
                        const float p = c[j] >= 0 ? s_lg[c[j] - cs][g] : 0.f;
                        st.l[g] -= p;
#pragma unroll
                        for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(-p, x[e], st.acc[g][e]);
                    }
                }
            }
        }
    } else if (a.pseudo) {
        // ---- waves 4-7: the approximate term of every cluster of the share --
#pragma unroll
        for (int j = 0; j < kPseudoDepth; ++j) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int c = cs + item(j, u);
                vload(pring[j].r[u], c < ce ? c : max(ce - 1, 0));
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // the weights, once per cluster and head, replace the logits in LDS (0
        // for clusters outside the share or empty), while the first rows fly;
        // their sum per head goes to the weight sum of lane 0 (the lane whose
        // sum the combine keeps), so the stream below only accumulates values
        float wsum[G];
#pragma unroll
        for (int g = 0; g < G; ++g) wsum[g] = 0.f;
        for (int t = tid - kCutWaves * kWave; t < kUnitShare; t += kStreamWaves * kWave) {
            const int c = cs + t;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float lgv = c < ce ? s_lg[t][g] : -INFINITY;
                const float w = lgv == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(lgv - Mref[g]);
                s_lg[t][g] = w;
                wsum[g] += w;
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float v = row16_sum(wsum[g]);
            v += shfl_xor_f(v, 16);
            v += shfl_xor_f(v, 32);
            if (lane == 0) st.l[g] += v;
        }
        int sgen = 0;
        group_barrier<kStreamWaves>(sctr, sgen);
        auto vconsume = [&](const VRows4& rr, int step) {
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = item(step, u);
                float x[8];
                rr.r[u].unpack(x);
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    const float w = s_lg[r][g];  // 0 past the share's clusters
#pragma unroll
                    for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(w, x[e], st.acc[g][e]);
                }
            }
        };
        // the last group is consumed without loading further rows (nothing
        // left in flight for the exact rows' first wait)
#pragma unroll 1
        for (int it = 0; it + kPseudoDepth < kSteps; it += kPseudoDepth) {
#pragma unroll
            for (int j = 0; j < kPseudoDepth; ++j) {
                vconsume(pring[j], it + j);
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    // rows past the share: its last row, or row 0 (cached)
                    const int c = cs + item(it + j + kPseudoDepth, u);
                    vload(pring[j].r[u], c < ce ? c : max(ce - 1, 0));
                }
                __builtin_amdgcn_sched_barrier(0);  // keep the ring order
            }
        }
#pragma unroll
        for (int j = 0; j < kPseudoDepth; ++j) vconsume(pring[j], kSteps - kPseudoDepth + j);
    }
    if (wave >= kCutWaves) {  // waves 4-7 join the exact rows once the first batch is staged
        while (__hip_atomic_load(rflag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == 0) __builtin_amdgcn_s_sleep(2);
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    }
    const int nsel = s_misc[6], E = s_misc[7];
    if (tid == 0 && a.dbg_exact && rep == 0) a.dbg_exact[unit] = E;

    // ---- exact rows of the replica's share, 16 rows per wave step through a
    //      ring of kExactDepth steps (branch-free body: exact wait counts; rows
    //      past the wave's range re-load cached rows and are masked).  The
    //      scores of a step come from the matrix cores (lane (rg, li)
    //      receives rows 4 rg + e for head li); the wave keeps one reference
    //      exponent per head, raised lazily as in SoftState; the weights go
    //      through a per-wave LDS tile to the row groups, which accumulate
    //      rows 4 rg + e of the step into their value sums.  The first batch
    //      starts on waves 0-3 as soon as they have staged it, while waves 4-7
    //      finish the approximate term, so waves 0-3 take the larger part of
    //      it; later batches (more than kUnitRowBatch rows per replica) are
    //      staged by all waves between workgroup barriers. -----------------
    const float qscale = kInvSqrtD * kLog2e;
    const size_t ubase = (size_t)su * a.Nmax * kHeadDim;
    int e0, e1;
    row_range(E, e0, e1);
    {
        const bf16_t* Kx = reinterpret_cast<const bf16_t*>(a.Kx) + ubase;
        const bf16_t* Vx = reinterpret_cast<const bf16_t*>(a.Vx) + ubase + li * 8;
        const bf16_t* Kt = reinterpret_cast<const bf16_t*>(a.K) + ubase;
        const bf16_t* Vt = reinterpret_cast<const bf16_t*>(a.V) + ubase + li * 8;
        QOperand qop;
        load_qop<G>(qop, qg, lane);
        // the wave's reference exponent of head li (entering: the same in
        // every row group) and the lane's weight sum of rows 4 rg + e, head li
        float mv = exact16_enter<G>(st);
        float lp = 0.f;
        float* sp = s_p + wave * 16 * G;  // [16][G] weights of the step
        // rows [w0, w1) of the staged batch, in order (the sums keep a fixed
        // order); rows past w1 re-load row w1 - 1 (a cache hit) and weigh
        // nothing
        auto run_rows = [&](int w0, int w1) {
            const int steps = (w1 - w0 + 15) / 16;
            auto row_at = [&](int i) { return s_row[max(min(i, w1 - 1), 0)]; };
            auto load_step = [&](ExactRows16& rr, int step) {
                const int ib = w0 + step * 16;
                const int rk = row_at(ib + li);
                load_row_blocks(rr.k, rk >= 0 ? Kx + (size_t)rk * kHeadDim : Kt + (size_t)(-1 - rk) * kHeadDim, lane);
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int rv = row_at(ib + 4 * rg + e);
                    rr.v[e].load(rv >= 0 ? Vx + (size_t)rv * kHeadDim : Vt + (size_t)(-1 - rv) * kHeadDim);
                }
            };
            ExactRows16 ring[kExactDepth];
#pragma unroll
            for (int j = 0; j < kExactDepth; ++j) {
                load_step(ring[j], j);
                __builtin_amdgcn_sched_barrier(0);
            }
            // the last group is consumed without loading further rows, so
            // nothing is in flight when the rows end (the combine that
            // follows would wait for it); with no rows at all its steps are
            // masked and weigh nothing
            int it = 0;
            for (; it + kExactDepth < steps; it += kExactDepth) {
#pragma unroll
                for (int j = 0; j < kExactDepth; ++j) {
                    exact16_step<G>(st, mv, lp, sp, qop, ring[j], w0 + (it + j) * 16 + 4 * rg, w1, qscale);
                    load_step(ring[j], it + j + kExactDepth);
                    __builtin_amdgcn_sched_barrier(0);  // keep the ring order
                }
            }
#pragma unroll
            for (int j = 0; j < kExactDepth; ++j)
                exact16_step<G>(st, mv, lp, sp, qop, ring[j], w0 + (it + j) * 16 + 4 * rg, w1, qscale);
        };
        // wave's contiguous part of `part` rows starting at `base`, shared by
        // the 4 waves of its half
        auto quarter = [&](int base, int part, int& w0, int& w1) {
            const int hw = wave & 3;
            w0 = base + part * hw / 4;
            w1 = base + part * (hw + 1) / 4;
        };
        {
            const int cnt = min(kUnitRowBatch, e1 - e0);
            const int na = (cnt * kFirstBatchEarly + 8) / 16;
            int w0, w1;
            if (wave < kCutWaves) quarter(0, na, w0, w1);
            else quarter(na, cnt - na, w0, w1);
            if (cnt > 0) run_rows(w0, w1);
        }
        for (int c0 = e0 + kUnitRowBatch; c0 < e1; c0 += kUnitRowBatch) {
            const int cnt = min(kUnitRowBatch, e1 - c0);
            lds_barrier();  // the previous batch is consumed
            stage(c0, cnt, nsel, E, tid, kUnitThreads);
            lds_barrier();
            // waves 0-3, which issue first on their SIMDs and were measured
            // to stream about a quarter faster than waves 4-7 beside them,
            // share the first 9/16 of the rows
            const int na = (cnt * 9 + 8) / 16;
            int w0, w1;
            if (wave < kCutWaves) quarter(0, na, w0, w1);
            else quarter(na, cnt - na, w0, w1);
            run_rows(w0, w1);
        }
        exact16_leave<G>(st, mv, lp);
    }
    if (wave < kCutWaves && a.pseudo) {  // the deferred first pass of the removal
#pragma unroll
        for (int g = 0; g < G; ++g) {
            // the weights are relative to Mref; the reference may have risen since
            const float sc = Mref[g] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(Mref[g] - st.m[g]);
#pragma unroll
            for (int j = 0; j < kRemoveBatch; ++j) rem_p[j][g] *= sc;
        }
#pragma unroll
        for (int j = 0; j < kRemoveBatch; ++j) {
            float x[8];
            rem_v[j].unpack(x);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                st.l[g] -= rem_p[j][g];
#pragma unroll
                for (int e = 0; e < 8; ++e) st.acc[g][e] = fmaf(-rem_p[j][g], x[e], st.acc[g][e]);
            }
        }
    }
    // The replicas count in on the unit's arrival counter as they enter the
    // combine, so the one that merges is the last to finish its rows: the
    // others' partials are posted (or nearly) when it reads them.  Counting
    // in right after the score pass instead picked the replica that finished
    // first about a third of the time, which then waited for its partner's
    // combine and post (measured 0.3-0.7 us slower per step).
    finish_step<G, kUnitWaves>(st, s_red, s_misc, a.out + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim,
                               a.xpart + (size_t)unit * R * G * (kHeadDim + 2), a.xcount + unit, tag,
                               R > 1 ? a.xepoch + unit : nullptr, a.status, R, rep, kPartialWaitTicks);
}

// One replica per unit only once the units alone give a workgroup to every CU
// (reading the key centroids twice costs less than leaving half the CUs idle).
int unit_replicas(int n_clusters, int units) {
    constexpr int kWorkgroups = 256;
    if (n_clusters <= kUnitMaxCSmall && units >= kWorkgroups) return 1;
    int r = (n_clusters + kUnitShareLarge - 1) / kUnitShareLarge;
    if (r < 2) r = 2;
    while (units * r < kWorkgroups && r < 8) ++r;
    return r;
}

bool unit_path_fits(int dtype, int G, int max_clusters) {
    return dtype == 1 && (G == 1 || G == 2 || G == 4 || G == 8) && max_clusters >= 1 && max_clusters <= kUnitMaxCLarge;
}

template <int MAXC, int SHARE, bool F8>
static hipError_t unit_dispatch_g(int G, const UnitArgs& a, dim3 grid, hipStream_t st) {
    switch (G) {
        case 1: hipLaunchKernelGGL((unit_decode_kernel<bf16_t, 1, MAXC, SHARE, F8>), grid, dim3(kUnitThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((unit_decode_kernel<bf16_t, 2, MAXC, SHARE, F8>), grid, dim3(kUnitThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL((unit_decode_kernel<bf16_t, 4, MAXC, SHARE, F8>), grid, dim3(kUnitThreads), 0, st, a); break;
        case 8: hipLaunchKernelGGL((unit_decode_kernel<bf16_t, 8, MAXC, SHARE, F8>), grid, dim3(kUnitThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int MAXC, int SHARE>
static hipError_t unit_dispatch(int G, const UnitArgs& a, dim3 grid, hipStream_t st) {
    return a.kcodes ? unit_dispatch_g<MAXC, SHARE, true>(G, a, grid, st)
                    : unit_dispatch_g<MAXC, SHARE, false>(G, a, grid, st);
}

hipError_t launch_unit_decode(int dtype, int G, const UnitArgs& a, int units, int replicas, hipStream_t st) {
    if (!unit_path_fits(dtype, G, a.C) || a.C > a.Cmax || replicas < 1 || a.ugroup < 1 ||
        !a.out || (replicas > 1 && (!a.xch || !a.xpart || !a.xcount || !a.xepoch)) ||
        (a.kcodes && (!a.kscales || !a.vcodes || !a.vscales)))
        return hipErrorInvalidValue;
    dim3 grid(units, replicas);
    if (replicas == 1) {
        if (a.C > kUnitShareSmall) return hipErrorInvalidValue;
        return unit_dispatch<kUnitMaxCSmall, kUnitShareSmall>(G, a, grid, st);
    }
    if ((a.C + replicas - 1) / replicas > kUnitShareLarge) return hipErrorInvalidValue;
    if (a.C <= kUnitMaxCSmall) return unit_dispatch<kUnitMaxCSmall, kUnitShareLarge>(G, a, grid, st);
    return unit_dispatch<kUnitMaxCLarge, kUnitShareLarge>(G, a, grid, st);
}

}  // namespace mpa
