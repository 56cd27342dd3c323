// dense.hip -- dense decode attention (every token exact) split over the
// tokens: the comparison point of the sparse decode.
//
// Pages: atlas.scime.ai summary, "Key results" (the speedups are quoted
// against a split-K dense decode, FlashDecoding, at batch 16 and 95%
// sparsity).
//
// Grid (splits, units).  A 256-thread workgroup streams the K/V rows of its
// token range in 16-row wave steps through a ring of kDenseDepth steps
// (scores on the matrix cores, the same step as the sparse decode's exact
// rows) and writes one partial (m, l, acc) per query head; the merge launch
// of decode.hip normalises.
#include <math.h>

#include "attn.hpp"
#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

constexpr int kDenseThreads = 256;
constexpr int kDenseWaves = kDenseThreads / kWave;  // 4
constexpr int kDenseDepth = 2;                      // 16-row steps in flight per wave

template <int G>
__global__ __launch_bounds__(kDenseThreads) void dense_kernel(DenseArgs a) {
    __shared__ float s_p[kDenseWaves][16 * G];
    __shared__ float s_red[kDenseWaves][G][kHeadDim + 2];
    const int split = blockIdx.x, unit = blockIdx.y, S = gridDim.x;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int b = unit / a.Hkv, h = unit % a.Hkv;
    // tokens [t0, t1) of this split, a multiple of 64 rows each
    const int per = ((a.n_tokens + S - 1) / S + 16 * kDenseWaves - 1) / (16 * kDenseWaves) * (16 * kDenseWaves);
    const int t0 = min(a.n_tokens, split * per), t1 = min(a.n_tokens, t0 + per);
    const int cnt = t1 - t0;
    const bf16_t* qg = reinterpret_cast<const bf16_t*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim;
    const size_t base = ((size_t)unit * a.Nmax + t0) * kHeadDim;
    const bf16_t* Ku = reinterpret_cast<const bf16_t*>(a.K) + base;
    const bf16_t* Vu = reinterpret_cast<const bf16_t*>(a.V) + base + li * 8;
    QOperand qop;
    load_qop<G>(qop, qg, lane);
    SoftState<G> st;
    st.init();
    float mv = exact16_enter<G>(st);
    float lp = 0.f;
    const float qscale = kInvSqrtD * kLog2e;
    auto load_step = [&](ExactRows16& rr, int step) {
        const int ib = step * 16 * kDenseWaves + wave * 16;
        const int ik = ib + li;
        load_row_blocks(rr.k, Ku + (size_t)(ik < cnt ? ik : 0) * kHeadDim, lane);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int iv = ib + 4 * rg + e;
            rr.v[e].load(Vu + (size_t)(iv < cnt ? iv : 0) * kHeadDim);
        }
    };
    if (cnt > 0) {  // uniform
        ExactRows16 ring[kDenseDepth];
#pragma unroll
        for (int j = 0; j < kDenseDepth; ++j) {
            load_step(ring[j], j);
            __builtin_amdgcn_sched_barrier(0);
        }
        const int steps = (cnt + 16 * kDenseWaves - 1) / (16 * kDenseWaves);
        for (int it = 0; it < steps; it += kDenseDepth) {
#pragma unroll
            for (int j = 0; j < kDenseDepth; ++j) {
                exact16_step<G>(st, mv, lp, s_p[wave], qop, ring[j], (it + j) * 16 * kDenseWaves + wave * 16 + 4 * rg,
                                cnt, qscale);
                load_step(ring[j], it + j + kDenseDepth);
                __builtin_amdgcn_sched_barrier(0);  // keep the ring order
            }
        }
    }
    exact16_leave<G>(st, mv, lp);
    // the row groups of a wave by shuffles, then the waves through LDS
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
    for (int e = tid; e < G * kHeadDim; e += kDenseThreads) {
        const int g = e / kHeadDim, dd = e % kHeadDim;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kDenseWaves; ++w) M = fmaxf(M, s_red[w][g][kHeadDim]);
        float l = 0.f, acc = 0.f;
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < kDenseWaves; ++w) {
                const float wt = __builtin_amdgcn_exp2f(s_red[w][g][kHeadDim] - M);
                l = fmaf(s_red[w][g][kHeadDim + 1], wt, l);
                acc = fmaf(s_red[w][g][dd], wt, acc);
            }
        }
        const size_t pidx = part_index(unit, G, g, S, split);
        a.part_acc[pidx * kHeadDim + dd] = acc;
        if (dd == 0) {
            a.part_ml[pidx * 2] = M;
            a.part_ml[pidx * 2 + 1] = l;
        }
    }
}

int dense_splits(int units) {
    int s = (1024 + units - 1) / units;  // about 1024 workgroups
    return s < 1 ? 1 : (s > 64 ? 64 : s);
}

hipError_t launch_dense(int G, const DenseArgs& a, int units, int splits, hipStream_t st) {
    if (!a.q || !a.K || !a.V || !a.part_ml || !a.part_acc || splits < 1 || a.n_tokens < 0) return hipErrorInvalidValue;
    const dim3 grid(splits, units);
    switch (G) {
        case 1: hipLaunchKernelGGL(dense_kernel<1>, grid, dim3(kDenseThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL(dense_kernel<2>, grid, dim3(kDenseThreads), 0, st, a); break;
        case 4: hipLaunchKernelGGL(dense_kernel<4>, grid, dim3(kDenseThreads), 0, st, a); break;
        case 8: hipLaunchKernelGGL(dense_kernel<8>, grid, dim3(kDenseThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace mpa
