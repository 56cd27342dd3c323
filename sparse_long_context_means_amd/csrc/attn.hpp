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
