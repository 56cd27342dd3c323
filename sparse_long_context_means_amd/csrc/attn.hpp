// attn.hpp -- device building blocks shared by the decode kernels: the
// order-preserving key of the budget cut, the online-softmax state of a
// 16-lane row group (base-2 exponents, fp32 sums) and the gathered exact-row
// steps.  Pages: atlas.scime.ai summary, opening sentence and "Approach"
// (exact attention on the selected clusters' keys, centroid terms for the
// rest).
#pragma once

#include <math.h>

#include "device.hpp"

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
// First pass of the budget cut, by value.  The cut keeps the longest prefix
// of the non-empty items in (key desc, id asc) order whose sizes fit the
// budget.  The open items' key range [min, max] is split into 256 bins of
// equal width; the bin index is a non-decreasing function of the key, so all
// items of a higher bin come before all items of a lower one.  A histogram
// of sizes (and counts) finds the bin where the budget runs out: items above
// it are taken, items below it dropped.  When at most kRankCap items share
// that bin (clustered keys put a handful there) each of them adds up the
// sizes of the bin's items ahead of it, by order key and id, and is taken if
// it still fits: the same decisions as an exact radix cut, in three barriers
// instead of six or more.  Otherwise, or when the key range is degenerate,
// it returns false with `act` holding the items still open and `budget` what
// is left of it, for an exact radix pass that starts with a barrier.
//
// Thread t holds ITEMS items (bit j of act / sel for its item j); id_of(j)
// is the id of its item j.  The NW waves 0 .. NW-1 take part, `bar` is their
// barrier.  h64: 256 64-bit words of histogram followed by kRankCap 16-byte
// list entries (LDS, 16-byte aligned); mm: 2 NW + 1 words (LDS).  Both are
// free again after the next barrier of the caller.
constexpr int kRankCap = 128;

template <int NW, int ITEMS, typename IdF, typename Bar>
__device__ __forceinline__ bool range_cut(const float (&kf)[ITEMS], const uint32_t (&key)[ITEMS],
                                          const int (&isz)[ITEMS], IdF id_of, int& budget, uint32_t& act,
                                          uint32_t& sel, unsigned long long* h64, float* mm, Bar bar) {
    static_assert(ITEMS <= 32, "one bit per item");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    uint4* s_list = reinterpret_cast<uint4*>(h64 + 256);
    int* s_cnt = reinterpret_cast<int*>(mm + 2 * NW);
    float lo = INFINITY, hi = -INFINITY;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
        if ((act >> j) & 1u) {
            lo = fminf(lo, kf[j]);
            hi = fmaxf(hi, kf[j]);
        }
#pragma unroll
    for (int o = kWave / 2; o >= 1; o >>= 1) {
        lo = fminf(lo, shfl_xor_f(lo, o));
        hi = fmaxf(hi, shfl_xor_f(hi, o));
    }
    if (lane == 0) {
        mm[2 * wave] = lo;
        mm[2 * wave + 1] = hi;
    }
    for (int k = tid; k < 256; k += NW * kWave) h64[k] = 0ull;
    if (tid == 0) *s_cnt = 0;
    bar();
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        lo = fminf(lo, mm[2 * w]);
        hi = fmaxf(hi, mm[2 * w + 1]);
    }
    const float width = hi - lo;
    if (!(width > 0.f) || !(width < INFINITY)) return false;  // the same in every thread
    const float inv = 256.f / width;
    int bin[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        bin[j] = (int)fminf(fmaxf((kf[j] - lo) * inv, 0.f), 255.f);
        if ((act >> j) & 1u) atomicAdd(&h64[bin[j]], (1ull << 40) | (unsigned long long)isz[j]);
    }
    bar();
    int vs[4], vc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const unsigned long long v = h64[255 - (4 * lane + q)];
        vs[q] = (int)(v & ((1ull << 40) - 1));
        vc[q] = (int)(v >> 40);
    }
    int total;
    int run = wave_exclusive_sum(vs[0] + vs[1] + vs[2] + vs[3], total);
    if (total <= budget) {  // every open item fits
        sel |= act;
        act = 0;
        return true;
    }
    int found = -1, cum = 0, cnt = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        if (found < 0 && run <= budget && budget < run + vs[q]) {
            found = 255 - (4 * lane + q);
            cum = run;
            cnt = vc[q];
        }
        run += vs[q];
    }
    const uint64_t bal = __ballot(found >= 0);
    const int src = __ffsll((long long)bal) - 1;
    const int c = lane_value(found, src), m = lane_value(cnt, src);
    budget -= lane_value(cum, src);
    uint32_t inbin = 0;
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
        if ((act >> j) & 1u) {
            if (bin[j] > c) sel |= 1u << j;
            else if (bin[j] == c) inbin |= 1u << j;
        }
    act = inbin;
    if (m > kRankCap) return false;
    // The bin's m items in a list (m counted them: the slots stay below m) as
    // 64-bit ranks (order key above, inverted id below: a larger rank comes
    // first) with their sizes.  Every wave then ranks the whole list, lane l
    // taking entries l and l + 64 against a broadcast of each entry; the
    // ballots of the two results give every owner its items' decisions.
    int slot[ITEMS];
#pragma unroll
    for (int j = 0; j < ITEMS; ++j) {
        slot[j] = -1;
        if ((inbin >> j) & 1u) {
            slot[j] = atomicAdd(s_cnt, 1);
            s_list[slot[j]] = make_uint4(~(uint32_t)id_of(j), key[j], (uint32_t)isz[j], 0u);
        }
    }
    bar();
    const uint4 e0 = lane < m ? s_list[lane] : make_uint4(0u, 0u, 0u, 0u);
    const uint4 e1 = lane + kWave < m ? s_list[lane + kWave] : make_uint4(0u, 0u, 0u, 0u);
    const uint64_t r0 = ((uint64_t)e0.y << 32) | e0.x, r1 = ((uint64_t)e1.y << 32) | e1.x;
    int b0 = 0, b1 = 0;
#pragma unroll 4
    for (int t = 0; t < m; ++t) {
        const uint4 e = s_list[t];
        const uint64_t r = ((uint64_t)e.y << 32) | e.x;
        b0 += r > r0 ? (int)e.z : 0;
        b1 += r > r1 ? (int)e.z : 0;
    }
    const uint64_t f0 = __ballot(lane < m && b0 + (int)e0.z <= budget);
    const uint64_t f1 = __ballot(lane + kWave < m && b1 + (int)e1.z <= budget);
#pragma unroll
    for (int j = 0; j < ITEMS; ++j)
        if (slot[j] >= 0 && (((slot[j] < kWave ? f0 : f1) >> (slot[j] & (kWave - 1))) & 1ull)) sel |= 1u << j;
    act = 0;
    return true;
}

// log2 of a positive count, as both the adding and the removing side take it.
__device__ __forceinline__ float log2_count(int n) { return __builtin_amdgcn_logf((float)n); }

// ---------------------------------------------------------------------------
// Online softmax state of a 16-lane row group: per query head g the reference
// exponent m, the sum l of 2^(logit - m) and the weighted value sum acc (the
// lane's 8 dimensions).  The reference is only raised when a logit exceeds it
// by more than 2^8 (every weight stays <= 256 in fp32), so rescaling is rare.
// ---------------------------------------------------------------------------
constexpr float kLazyMax = 8.0f;

template <int G>
struct SoftState {
    float m[G], l[G], acc[G][8];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            m[g] = -INFINITY;
            l[g] = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[g][e] = 0.f;
        }
    }
};

// Adds (NEG: removes) 2 rows with base-2 logits lg[u][g] (-inf: absent row).
template <typename T, int G, bool NEG>
__device__ __forceinline__ void absorb2(SoftState<G>& st, const float (&lg)[2][G], const Slice8<T> (&v)[2]) {
    float x0[8], x1[8];
    v[0].unpack(x0);
    v[1].unpack(x1);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mx = fmaxf(lg[0][g], lg[1][g]);
        if (mx == -INFINITY) continue;
        if (mx > st.m[g] + kLazyMax) {  // rare: raise the reference
            const float sc = __builtin_amdgcn_exp2f(st.m[g] - mx);
            st.l[g] *= sc;
#pragma unroll
            for (int e = 0; e < 8; ++e) st.acc[g][e] *= sc;
            st.m[g] = mx;
        }
        float p0 = __builtin_amdgcn_exp2f(lg[0][g] - st.m[g]);
        float p1 = __builtin_amdgcn_exp2f(lg[1][g] - st.m[g]);
        if (NEG) {
            p0 = -p0;
            p1 = -p1;
        }
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

// Partial (m, l, acc) of query head g of a unit in slot `slot` of P.
__device__ __forceinline__ size_t part_index(int unit, int G, int g, int P, int slot) {
    return ((size_t)unit * G + g) * P + slot;
}

// ---------------------------------------------------------------------------
// Scores on the matrix cores: v_mfma_f32_16x16x32_bf16 multiplies 16 key rows
// (A: lane l holds row l % 16, dimensions 32 kk + 8 (l / 16) .. + 8 of k-block
// kk) by the query heads of a group (B: lane l holds head l % 16 at the same
// dimensions, zero for heads >= G); lane l receives the dot products of rows
// 4 (l / 16) + i, i < 4, with head l % 16.  Four k-blocks cover d = 128.
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8v;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4v;
typedef __attribute__((ext_vector_type(2))) float f32x2v;

struct QOperand {
    uint4 b[4];
};

// qg: head 0 of the group, [G][d] contiguous.
template <int G>
__device__ __forceinline__ void load_qop(QOperand& q, const bf16_t* qg, int lane) {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        q.b[kk] = n < G ? *reinterpret_cast<const uint4*>(qg + (size_t)n * kHeadDim + kk * 32 + grp * 8)
                        : make_uint4(0u, 0u, 0u, 0u);
}

// The lane's share of its row (row l % 16 of the 16): 4 loads of 16 bytes.
__device__ __forceinline__ void load_row_blocks(Slice8<bf16_t> (&a)[4], const bf16_t* row, int lane) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) a[kk].load(row + kk * 32 + (lane >> 4) * 8);
}

__device__ __forceinline__ f32x4v mfma_scores(const Slice8<bf16_t> (&a)[4], const QOperand& q) {
    f32x4v d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8v, a[kk].raw),
                                                    __builtin_bit_cast(bf16x8v, q.b[kk]), d, 0, 0, 0);
    return d;
}

// ---------------------------------------------------------------------------
// fp8 centroid copies: E4M3 codes with one scale byte (E + 127) per 32
// values of a row.  The gfx950 scaled conversions decode code x 2^E exactly
// (they take the exponent of the scale operand; 2^E is a normal float since
// the byte is 1 .. 254).
__device__ __forceinline__ float code_scale(uint32_t byte) { return __uint_as_float(byte << 23); }

// Score operand of a coded key-centroid row.  Lane (row l % 16, group l / 16)
// holds the 32 codes of block l / 16 (one scale); operand kk is codes
// 8 kk .. 8 kk + 7 of them, so the query operand must take its elements in
// the same order (load_qop_blocks).
struct KCodes {
    uint4 lo, hi;
    uint32_t sc;
    __device__ __forceinline__ void load(const uint8_t* codes_row, const uint8_t* scales_row, int grp) {
        lo = *reinterpret_cast<const uint4*>(codes_row + grp * 32);
        hi = *reinterpret_cast<const uint4*>(codes_row + grp * 32 + 16);
        sc = scales_row[grp];
    }
    __device__ __forceinline__ void operands(Slice8<bf16_t> (&a)[4]) const {
        const float s = code_scale(sc);
        const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            a[kk].raw.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * kk], s, false));
            a[kk].raw.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * kk], s, true));
            a[kk].raw.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * kk + 1], s, false));
            a[kk].raw.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 * kk + 1], s, true));
        }
    }
};

// Query operand in the order of KCodes: operand kk of lane (n, grp) holds
// elements 32 grp + 8 kk .. + 7 of head n.
template <int G>
__device__ __forceinline__ void load_qop_blocks(QOperand& q, const bf16_t* qg, int lane) {
    const int n = lane & 15, grp = lane >> 4;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        q.b[kk] = n < G ? *reinterpret_cast<const uint4*>(qg + (size_t)n * kHeadDim + grp * 32 + kk * 8)
                        : make_uint4(0u, 0u, 0u, 0u);
}

// Eight consecutive values of a coded value-centroid row (one scale).
struct VCodes8 {
    uint2 raw;
    uint32_t sc;
    __device__ __forceinline__ void load(const uint8_t* codes, const uint8_t* scale) {
        raw = *reinterpret_cast<const uint2*>(codes);
        sc = *scale;
    }
    __device__ __forceinline__ void unpack(float* x) const {
        const float s = code_scale(sc);
        const f32x2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, s, false);
        const f32x2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.x, s, true);
        const f32x2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, s, false);
        const f32x2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(raw.y, s, true);
        x[0] = p0[0]; x[1] = p0[1]; x[2] = p1[0]; x[3] = p1[1];
        x[4] = p2[0]; x[5] = p2[1]; x[6] = p3[0]; x[7] = p3[1];
    }
};

// Mean of a row's scores over the G heads (lanes l % 16 < G); the result is
// valid in lanes with l % 16 == 0.  The same operations on every path give
// the same ranking keys.
template <int G>
__device__ __forceinline__ float head_mean(float s) {
    if (G >= 2) s += MPA_DPP(s, 0xB1);   // quad_perm [1,0,3,2]
    if (G >= 4) s += MPA_DPP(s, 0x4E);   // quad_perm [2,3,0,1]
    if (G >= 8) s += MPA_DPP(s, 0x141);  // row_half_mirror: lane 0 takes lane 7
    return s * (1.0f / G);
}

// ---------------------------------------------------------------------------
// Exact rows on the matrix cores, 16 per wave step.  Lane l loads the blocks
// of key row l % 16 (the A operand) and the 8-element slices of value rows
// 4 (l / 16) + e (e < 4), so row group l / 16 accumulates those four rows.  The
// wave keeps one reference exponent per head (mv in lane l for head l % 16,
// the same in every row group, raised lazily as in SoftState) and each lane
// the weight sum lp of its rows 4 (l / 16) + e for head l % 16; the weights
// reach the row groups through a per-wave LDS tile sp[16][G].
// ---------------------------------------------------------------------------
struct ExactRows16 {
    Slice8<bf16_t> k[4], v[4];
};

// Matrix-core form of the state on entry (st.m the same in every row group).
template <int G>
__device__ __forceinline__ float exact16_enter(const SoftState<G>& st) {
    const int li = threadIdx.x & 15;
    float mv = 0.f;
#pragma unroll
    for (int g = 0; g < G; ++g) mv = li == g ? st.m[g] : mv;
    return mv;
}

// One step: rows first_row + e (e < 4) of row group l / 16 count while below
// `cnt`; the others weigh nothing.
template <int G>
__device__ __forceinline__ void exact16_step(SoftState<G>& st, float& mv, float& lp, float* sp, const QOperand& qop,
                                             const ExactRows16& rr, int first_row, int cnt, float qscale) {
    const int lane = threadIdx.x & (kWave - 1), rg = lane >> 4, li = lane & 15;
    const f32x4v d = mfma_scores(rr.k, qop);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        sv[e] = first_row + e < cnt ? d[e] * qscale : -INFINITY;
        mx = fmaxf(mx, sv[e]);
    }
    mx = fmaxf(mx, shfl_xor_f(mx, 16));
    mx = fmaxf(mx, shfl_xor_f(mx, 32));
    const bool raise = li < G && mx > mv + kLazyMax;
    if (__builtin_amdgcn_ballot_w64(raise)) {  // rare, wave-uniform
        const float sc = raise ? __builtin_amdgcn_exp2f(mv - mx) : 1.f;
        mv = raise ? mx : mv;
        lp *= sc;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float sg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sc), g));
            st.l[g] *= sg;
#pragma unroll
            for (int x = 0; x < 8; ++x) st.acc[g][x] *= sg;
        }
    }
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        pe[e] = sv[e] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sv[e] - mv);
        lp += pe[e];
    }
    if (li < G) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sp[(4 * rg + e) * G + li] = pe[e];
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float pg[G];
#pragma unroll
        for (int g = 0; g < G; ++g) pg[g] = sp[(4 * rg + e) * G + g];
        float x[8];
        rr.v[e].unpack(x);
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 8; ++q) st.acc[g][q] = fmaf(pg[g], x[q], st.acc[g][q]);
    }
    __builtin_amdgcn_wave_barrier();
}

// Back to the row-group form: the wave's reference, the row groups' sums.
template <int G>
__device__ __forceinline__ void exact16_leave(SoftState<G>& st, float mv, float lp) {
    const int rg = (threadIdx.x & (kWave - 1)) >> 4;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        st.m[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mv), g));
        st.l[g] += __shfl(lp, rg * 16 + g, kWave);
    }
}

// ---------------------------------------------------------------------------
// Workgroup barrier ordering LDS only: global loads and stores in flight are
// not waited for (every barrier of the one-launch kernels publishes LDS data;
// a plain __syncthreads() after a global store would also drain the load
// rings).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// End of a unit's step in a workgroup of NW waves (one-launch kernels): the
// row groups' states are combined (shuffles), then the waves' (through
// s_red, which may alias LDS data that is dead once every wave got here).
// With one workgroup per unit (R = 1) it writes the normalised output outu
// [G][d].  Otherwise each of the R workgroups counts itself in on the unit's
// arrival counter *xcount as it enters; all but the last to arrive post their partial (per head the state m, l and the 128 sums) as words (tag <<
// 32 | value) into their slot of xp [R][G][d + 2] and are done.  The last
// one reads the others' partials -- polling a word that still carries
// another call's tag for at most wait_ticks of the 100 MHz constant clock (a
// word given up on is counted in status[1], status may be null) -- merges
// them in workgroup order, sets the counter back to zero and stores the
// call's tag in the unit's *epoch.  s_flag: one int of LDS that nothing else
// uses during the call.
template <int G, int NW>
__device__ __forceinline__ void finish_step(SoftState<G>& st, float (*s_red)[G][kHeadDim + 2], int* s_flag,
                                            float* outu, uint64_t* xp, uint64_t* xcount, uint32_t tag,
                                            uint32_t* epoch, uint32_t* status, int R, int rep,
                                            uint64_t wait_ticks) {
    constexpr int kThreads = NW * kWave;
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int rg = lane >> 4, li = lane & 15;
    const uint64_t tagw = (uint64_t)tag << 32;
    // several replicas: count in on the unit's arrival counter now, so the
    // round trip runs beside the combine below (the replica that sees R - 1
    // arrivals before its own merges; it finds the others' partials by their
    // tags, polling while a partner still stores them)
    if (R > 1 && tid == 0) {
        const uint64_t arrivals = __hip_atomic_fetch_add(xcount, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_flag = arrivals + 1 == (uint64_t)R;  // read after the barriers below
    }
    // ---- combine the row groups, 4 per wave, then the waves through LDS (in
    //      wave order).  When the row groups of the wave share each head's
    //      reference exponent (the exact-row steps keep one per wave) their
    //      sums just add, four values at a time: v_permlane16_swap of two
    //      values adds pairs of rows of both (a in rows 0 and 2, b in rows 1
    //      and 3), v_permlane32_swap of two such results adds the halves, and
    //      row group k ends up with the wave's total of the k-th value.  These
    //      are the additions of the general merge below, in its order, which
    //      shuffles through LDS and leaves every total in row group 0. -------
    bool uniform = true;
#pragma unroll
    for (int g = 0; g < G; ++g)
        uniform = uniform && __builtin_amdgcn_ballot_w64(st.m[g] != __int_as_float(__builtin_amdgcn_readlane(
                                                             __float_as_int(st.m[g]), 0))) == 0;
    auto quad_sum = [](float a, float b, float c, float d) {
        const auto r1 = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
        const float s1 = __uint_as_float(r1[0]) + __uint_as_float(r1[1]);
        const auto r2 = __builtin_amdgcn_permlane16_swap(__float_as_uint(c), __float_as_uint(d), false, false);
        const float s2 = __uint_as_float(r2[0]) + __uint_as_float(r2[1]);
        const auto r3 = __builtin_amdgcn_permlane32_swap(__float_as_uint(s1), __float_as_uint(s2), false, false);
        return __uint_as_float(r3[0]) + __uint_as_float(r3[1]);
    };
    constexpr int kLq = G % 4 == 0 ? G / 4 : 0;  // quadruples of heads for the weight sums
    float qacc[G][2];                             // row group rg: dimension li * 8 + 4 q + rg
    float ql[kLq > 0 ? kLq : 1];                  // row group rg: head 4 j + rg
    if (uniform) {  // (wave-uniform)
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 2; ++q)
                qacc[g][q] = quad_sum(st.acc[g][4 * q], st.acc[g][4 * q + 1], st.acc[g][4 * q + 2], st.acc[g][4 * q + 3]);
        if constexpr (kLq > 0) {
#pragma unroll
            for (int j = 0; j < kLq; ++j)
                ql[j] = quad_sum(st.l[4 * j], st.l[4 * j + 1], st.l[4 * j + 2], st.l[4 * j + 3]);
        } else {  // one or two heads: the weight sums of every row group, one at a time
#pragma unroll
            for (int g = 0; g < G; ++g) {
                auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(st.l[g]), __float_as_uint(st.l[g]), false, false);
                st.l[g] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
                r = __builtin_amdgcn_permlane32_swap(__float_as_uint(st.l[g]), __float_as_uint(st.l[g]), false, false);
                st.l[g] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
            }
        }
    } else {
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
    }
    lds_barrier();  // the big region is free
    if (uniform) {
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int q = 0; q < 2; ++q) s_red[wave][g][li * 8 + 4 * q + rg] = qacc[g][q];
        if (li == 0) {
            if constexpr (kLq > 0) {
                if (rg == 0) {
#pragma unroll
                    for (int g = 0; g < G; ++g) s_red[wave][g][kHeadDim] = st.m[g];
                }
#pragma unroll
                for (int j = 0; j < kLq; ++j) s_red[wave][4 * j + rg][kHeadDim + 1] = ql[j];
            } else if (rg == 0) {
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    s_red[wave][g][kHeadDim] = st.m[g];
                    s_red[wave][g][kHeadDim + 1] = st.l[g];
                }
            }
        }
    } else if (rg == 0) {
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
    lds_barrier();
    // thread tid owns outputs e = tid + kThreads k of the unit's G heads
    constexpr int kOut = (G * kHeadDim + kThreads - 1) / kThreads;
    float oM[kOut], oL[kOut], oA[kOut];
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
        const int e = tid + k * kThreads;
        if (e >= G * kHeadDim) break;
        const int g = e / kHeadDim, dd = e % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, s_red[w][g][kHeadDim]);
        float l = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const float wt = __builtin_amdgcn_exp2f(s_red[w][g][kHeadDim] - M);
                l = fmaf(s_red[w][g][kHeadDim + 1], wt, l);
                acc = fmaf(s_red[w][g][dd], wt, acc);
            }
        }
        oM[k] = M;
        oL[k] = l;
        oA[k] = acc;
    }
    if (R == 1) {
#pragma unroll
        for (int k = 0; k < kOut; ++k) {
            const int e = tid + k * kThreads;
            if (e < G * kHeadDim) outu[e] = oL[k] > 0.f ? oA[k] / oL[k] : 0.f;
        }
        return;
    }

    // ---- several replicas: the others each post their partial (per head:
    //      the state m, l and the 128 sums) as tagged words and are done; the
    //      replica that counted in last stores nothing (its own stores would
    //      hold up its loads, which complete after them) and reads the others'
    //      partials, then writes the normalised output, merging in replica
    //      order. ------------------------------------------------------------
    constexpr int kPart = G * (kHeadDim + 2);
    if (!*s_flag) {
#pragma unroll
        for (int k = 0; k < kOut; ++k) {
            const int e = tid + k * kThreads;
            if (e >= G * kHeadDim) break;
            const int g = e / kHeadDim, dd = e % kHeadDim;
            uint64_t* pg = xp + (size_t)rep * kPart + g * (kHeadDim + 2);
            __hip_atomic_store(pg + dd, tagw | __float_as_uint(oA[k]), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (dd == 0) {
                __hip_atomic_store(pg + kHeadDim, tagw | __float_as_uint(oM[k]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(pg + kHeadDim + 1, tagw | __float_as_uint(oL[k]), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        return;
    }
    constexpr int kMaxR = 8;
    uint64_t wm[kOut][kMaxR], wl[kOut][kMaxR], wa[kOut][kMaxR];
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
        const int e = tid + k * kThreads;
        if (e >= G * kHeadDim) break;
        const int g = e / kHeadDim, dd = e % kHeadDim;
#pragma unroll
        for (int r2 = 0; r2 < kMaxR; ++r2) {
            if (r2 < R && r2 != rep) {
                const uint64_t* pg = xp + (size_t)r2 * kPart + g * (kHeadDim + 2);
                wm[k][r2] = __hip_atomic_load(pg + kHeadDim, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                wl[k][r2] = __hip_atomic_load(pg + kHeadDim + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                wa[k][r2] = __hip_atomic_load(pg + dd, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    const uint64_t t0 = wall_clock64();
    bool late = false;
    // a partner word of this call (polled again, for a bounded time, while it
    // still carries another call's tag)
    auto fresh = [&](uint64_t v, const uint64_t* p) {
        while ((uint32_t)(v >> 32) != tag && !late) {
            if (wall_clock64() - t0 > wait_ticks) late = true;
            __builtin_amdgcn_s_sleep(1);
            v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        return (uint32_t)(v >> 32) == tag ? __uint_as_float((uint32_t)v) : NAN;
    };
#pragma unroll
    for (int k = 0; k < kOut; ++k) {
        const int e = tid + k * kThreads;
        if (e >= G * kHeadDim) break;
        const int g = e / kHeadDim, dd = e % kHeadDim;
        float pm[kMaxR], pl[kMaxR], pa[kMaxR];
        float M = -INFINITY;
#pragma unroll
        for (int r2 = 0; r2 < kMaxR; ++r2) {
            if (r2 < R) {
                if (r2 == rep) {
                    pm[r2] = oM[k];
                    pl[r2] = oL[k];
                    pa[r2] = oA[k];
                } else {
                    const uint64_t* pg = xp + (size_t)r2 * kPart + g * (kHeadDim + 2);
                    pm[r2] = fresh(wm[k][r2], pg + kHeadDim);
                    pl[r2] = fresh(wl[k][r2], pg + kHeadDim + 1);
                    pa[r2] = fresh(wa[k][r2], pg + dd);
                }
                M = fmaxf(M, pm[r2]);
            }
        }
        float l = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int r2 = 0; r2 < kMaxR; ++r2) {
                if (r2 < R) {
                    const float wt = __builtin_amdgcn_exp2f(pm[r2] - M);
                    l = fmaf(pl[r2], wt, l);
                    acc = fmaf(pa[r2], wt, acc);
                }
            }
        }
        // a partial that has not arrived within the bounded wait poisons the
        // output instead of hanging, and is counted in status[1]
        outu[e] = late ? NAN : (l > 0.f ? acc / l : 0.f);
        if (late && status) __hip_atomic_fetch_add(status + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // the merging replica is the last of the unit: every replica has counted
    // in and read the unit's epoch, so the counter starts again from zero and
    // the next decode takes the following tag
    if (tid == 0) {
        __hip_atomic_store(xcount, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *epoch = tag;
    }
}

template <typename T>
struct RowBuf {
    Slice8<T> k[2], v[2];
    bool ok[2];
};

// Loads rows it * (8 W) + wave * 8 + u * 4 + rg (u = 0, 1) of a staged list
// (W waves; 2 rows per row group and step).
template <typename T>
__device__ __forceinline__ void load_rows(RowBuf<T>& bf, const int32_t* s_row, int cnt, int it, int wave, int rg,
                                          const T* Kx, const T* Vx, int waves = 4) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = it * 8 * waves + wave * 8 + u * 4 + rg;
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
    absorb2<T, G, false>(st, lg, bf.v);
}

// Stages exact rows [c0, c0 + cnt) of the unit's selection: row i belongs to
// selected cluster k with pre[k] <= i < pre[k + 1] and sits at member position
// off[k] + i - pre[k] (through token ids when rows are gathered from K/V).
__device__ __forceinline__ void stage_exact(int32_t* s_row, const int32_t* pre, const int32_t* off, int nsel,
                                            const int32_t* tids, int c0, int cnt) {
    for (int i = threadIdx.x; i < cnt; i += blockDim.x) {
        const int r = c0 + i;
        const int k = upper_index(pre, nsel, r);
        const int pos = off[k] + r - pre[k];
        s_row[i] = tids ? tids[pos] : pos;
    }
}

}  // namespace mpa
