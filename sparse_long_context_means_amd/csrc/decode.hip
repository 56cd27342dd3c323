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
//   score  -- s[c][g] = q_g . Kbar_c / sqrt(d) and the group-mean ranking key;
//   select -- one wave per unit takes the budget cut (longest prefix of the
//             (key desc, id asc) order whose sizes fit the budget) with a radix
//             select and writes the exact row positions and the list of
//             approximated clusters;
//   attend -- split-K online softmax over exact rows (gathered K/V), the
//             unclustered tail and the approximated clusters (logit s + ln n,
//             value Vbar), in base-2 exponent units, fp32 partials;
//   merge  -- log-sum-exp merge of the splits.
// Kernel boundaries carry the cross-workgroup dependencies: a device-scope
// fence per workgroup (write back + invalidate of an XCD's L2) serialises and
// costs far more than a launch on this chip.
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

// ---------------------------------------------------------------------------
// score: workgroup (chunk, unit) scores 256 items, 16 lanes per centroid row,
// 8 rows per lane group in flight, two passes.
// select: one wave per unit (separate launch: the kernel boundary makes every
// score visible to it across XCDs).
// ---------------------------------------------------------------------------
constexpr int kScoreChunk = 256;  // items per workgroup (64 per wave)
constexpr int kSelCap = 2048;     // items staged in LDS for the cut
constexpr int kSelPad = kSelCap + kSelCap / 32;  // one pad word per 32 items

// LDS slot of item t: lane l reads items 32 l .. 32 l + 31, so one pad word
// per 32 items puts the 64 lanes of a wave on distinct banks.
__device__ __forceinline__ int sel_slot(int t) { return t + (t >> 5); }
constexpr int kSelTile = 2048;    // items per lane-tile pass (32 consecutive items per lane)

__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0;  // -0 ranks as +0
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Orders LDS and memory accesses of this wave before the following ones.
__device__ __forceinline__ void wave_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "workgroup");
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ int wave_exclusive_sum(int v, int& total) {
    const int inc = wave_inclusive_sum(v);
    total = __shfl(inc, kWave - 1, kWave);
    return inc - v;
}

// Budget cut of one unit by a single wave (lane = threadIdx.x < 64).
// Items t in [0, n): key, size and start offset (through ids when present).
// Four 8-bit radix passes over the order-preserving key bits find the cut
// value: the size-weighted histogram of the items still matching the prefix
// is scanned from the top digit down until the budget left is crossed.
// Items above the cut value are selected; items equal to it are taken in
// item order while they fit.  Then, in item order: positions of the exact
// rows, the list of approximated clusters and the counts.
template <bool kLds>
__device__ __forceinline__ void select_wave(const SelectArgs& a, int unit, int n, float* s_key, int32_t* s_size, int32_t* s_off,
                            int32_t* s_end, int32_t* s_id, int* hist) {
    const int lane = threadIdx.x & (kWave - 1);
    const float* gkey = a.key + (size_t)unit * a.key_stride;
    const int32_t* gids = a.ids ? a.ids + (size_t)unit * a.key_stride : nullptr;
    const int32_t* gsz = a.sizes + (size_t)unit * a.size_stride;
    const int32_t* goff = a.offsets + (size_t)unit * (a.size_stride + 1);
    if (kLds) {
        for (int t = lane; t < n; t += kWave) {
            const int id = gids ? gids[t] : t;
            const int sl = sel_slot(t);
            s_key[sl] = gkey[t];
            s_id[sl] = id;
            s_size[sl] = gsz[id];
            s_off[sl] = goff[id];
            s_end[sl] = goff[id + 1];
        }
        wave_sync();
    }
    auto KEY = [&](int t) { return kLds ? s_key[sel_slot(t)] : gkey[t]; };
    auto ID = [&](int t) { return kLds ? s_id[sel_slot(t)] : (gids ? gids[t] : t); };
    auto SIZE = [&](int t) { return kLds ? s_size[sel_slot(t)] : gsz[gids ? gids[t] : t]; };
    auto OFF = [&](int t) { return kLds ? s_off[sel_slot(t)] : goff[gids ? gids[t] : t]; };
    auto END = [&](int t) { return kLds ? s_end[sel_slot(t)] : goff[(gids ? gids[t] : t) + 1]; };

    uint32_t prefix = 0, mask = 0;
    int R = a.budget;
    bool done = false;
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int j = 0; j < 4; ++j) hist[4 * lane + j] = 0;
        wave_sync();
        for (int base = 0; base < n; base += kSelTile) {
            for (int k = 0; k < 32; ++k) {
                const int t = base + lane * 32 + k;
                if (t < n) {
                    const int sz = SIZE(t);
                    if (sz > 0) {
                        const uint32_t u = order_key(KEY(t));
                        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], sz);
                    }
                }
            }
        }
        wave_sync();
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = hist[255 - (4 * lane + j)];
        int total;
        int run = wave_exclusive_sum(v[0] + v[1] + v[2] + v[3], total);
        if (total <= R) {  // uniform across the wave
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
        const int digit = __shfl(found, src, kWave);
        R -= __shfl(cum, src, kWave);
        prefix |= (uint32_t)digit << shift;
        mask |= 0xFFu << shift;
        wave_sync();
    }
    const uint32_t tau = prefix;

    int32_t* rows = a.rows + (size_t)unit * a.row_stride;
    int32_t* plist = a.plist + (size_t)unit * a.plist_stride;
    int32_t* dbg = a.dbg_selected ? a.dbg_selected + (size_t)unit * a.dbg_stride : nullptr;
    int carry_tie = 0, carry_rows = 0, carry_p = 0, carry_sel = 0;
    for (int base = 0; base < n; base += kSelTile) {
        int tie_local = 0;
        if (!done) {
            for (int k = 0; k < 32; ++k) {
                const int t = base + lane * 32 + k;
                if (t < n) {
                    const int sz = SIZE(t);
                    if (sz > 0 && order_key(KEY(t)) == tau) tie_local += sz;
                }
            }
        }
        int tie_total;
        int run_tie = carry_tie + wave_exclusive_sum(tie_local, tie_total);
        uint32_t selbits = 0;
        int rows_local = 0, p_local = 0, s_local = 0;
        for (int k = 0; k < 32; ++k) {
            const int t = base + lane * 32 + k;
            if (t >= n) break;
            const int sz = SIZE(t);
            if (sz <= 0) continue;
            const uint32_t u = order_key(KEY(t));
            bool sel;
            if (done) {
                sel = u >= prefix;
            } else {
                const bool tie = u == tau;
                sel = u > tau || (tie && run_tie + sz <= R);
                if (tie) run_tie += sz;
            }
            if (sel) {
                selbits |= 1u << k;
                rows_local += END(t) - OFF(t);
                ++s_local;
            } else if (a.want_pseudo) {
                ++p_local;
            }
        }
        int rt, pt, st;
        int ro = carry_rows + wave_exclusive_sum(rows_local, rt);
        int po = carry_p + wave_exclusive_sum(p_local, pt);
        wave_exclusive_sum(s_local, st);
        for (int k = 0; k < 32; ++k) {
            const int t = base + lane * 32 + k;
            if (t >= n) break;
            const int sz = SIZE(t);
            const int id = ID(t);
            const bool sel = (selbits >> k) & 1u;
            if (sel) {
                const int off = OFF(t), nr = END(t) - off;
                for (int jx = 0; jx < nr; ++jx) rows[ro + jx] = off + jx;
                ro += nr;
            } else if (sz > 0 && a.want_pseudo) {
                plist[po++] = id;
            }
            if (dbg) dbg[id] = sel ? 1 : 0;
        }
        carry_tie += tie_total;
        carry_rows += rt;
        carry_p += pt;
        carry_sel += st;
    }
    if (lane == 0) {
        int32_t* cnt = a.counts + unit * 4;
        cnt[0] = carry_rows;
        cnt[1] = carry_p;
        cnt[2] = carry_sel;
        cnt[3] = 0;
    }
}

template <typename T, int G>
__global__ __launch_bounds__(256) void score_kernel(ScoreArgs a) {
    const int unit = blockIdx.y;
    int n = a.n_items;
    if (a.n_items_dev) n = min(n, a.n_items_dev[unit * 4]);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int i0 = blockIdx.x * kScoreChunk + wave * 64;

    if (i0 < n) {
        const int b = unit / a.Hkv, h = unit % a.Hkv;
        float qv[G][8];
        const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            Slice8<T> s;
            s.load(qb + (size_t)g * kHeadDim);
            s.unpack(qv[g]);
        }
        const T* cu = reinterpret_cast<const T*>(a.cent) + (size_t)unit * a.cent_rows * kHeadDim + li * 8;
        const int32_t* pl = a.pos_list ? a.pos_list + (size_t)unit * a.list_stride : nullptr;
        const int32_t* mem = a.members ? a.members + (size_t)unit * a.cent_rows : nullptr;
#pragma unroll 1
        for (int half = 0; half < 2; ++half) {  // 2 x 8 rows per lane group in flight
            const int ib = i0 + half * 32;
            int cid[8];
            Slice8<T> row[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = ib + u * 4 + rg;
                const int ii = i < n ? i : i0;
                cid[u] = pl ? mem[pl[ii]] : ii;
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) row[u].load(cu + (size_t)cid[u] * kHeadDim);
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int i = ib + u * 4 + rg;
                float x[8];
                row[u].unpack(x);
                float sg[G];
                float r = 0.f;
#pragma unroll
                for (int g = 0; g < G; ++g) {
                    float d = qv[g][0] * x[0];
#pragma unroll
                    for (int e = 1; e < 8; ++e) d = fmaf(qv[g][e], x[e], d);
                    sg[g] = row16_sum(d) * kInvSqrtD;
                    r += sg[g];
                }
                r *= 1.0f / G;
                if (i < n) {
                    float* so = a.s_out + ((size_t)unit * a.cent_rows + cid[u]) * G;
                    float mine = sg[0];
#pragma unroll
                    for (int g = 1; g < G; ++g) mine = li == g ? sg[g] : mine;
                    if (li < G) so[li] = mine;
                    if (li == G) a.r_out[(size_t)unit * a.r_stride + i] = r;
                    if (a.ids_out && li == 15) a.ids_out[(size_t)unit * a.r_stride + i] = cid[u];
                }
            }
        }
    }
}

// One wave per unit takes the budget cut.
__global__ __launch_bounds__(64) void select_kernel(SelectArgs se) {
    __shared__ float s_key[kSelPad];
    __shared__ int32_t s_size[kSelPad];
    __shared__ int32_t s_off[kSelPad];
    __shared__ int32_t s_end[kSelPad];
    __shared__ int32_t s_id[kSelPad];
    __shared__ int hist[256];
    const int unit = blockIdx.x;
    int n = se.n_items;
    if (se.n_items_dev) n = min(n, se.n_items_dev[unit * 4]);
    if (n <= kSelCap)
        select_wave<true>(se, unit, n, s_key, s_size, s_off, s_end, s_id, hist);
    else
        select_wave<false>(se, unit, n, s_key, s_size, s_off, s_end, s_id, hist);
}

// ---------------------------------------------------------------------------
// attend: workgroup (split, unit), 4 waves, 16 lanes per row.  Each row group
// (16 lanes) keeps its own online-softmax state (m, l, acc[8] per head) over
// the rows it visits, 4 rows per step; the 4 row groups of a wave and the 4
// waves are merged at the end.  Index lists of the split are staged in LDS;
// row loads of the next step are issued before the current step's math.
// ---------------------------------------------------------------------------
constexpr int kAttCap = 512;  // staged indices per list and pass

template <int G>
struct SoftState {
    float m[G], l[G], acc[G][8];
};

template <typename T, int G>
__device__ __forceinline__ void absorb4(SoftState<G>& st, const float (&lg)[4][G], const Slice8<T> (&v)[4]) {
    float x[4][8];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u].unpack(x[u]);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float mx = fmaxf(fmaxf(lg[0][g], lg[1][g]), fmaxf(lg[2][g], lg[3][g]));
        const float mnew = fmaxf(st.m[g], mx);
        if (mnew == -INFINITY) continue;
        const float sc = __builtin_amdgcn_exp2f(st.m[g] - mnew);
        float p[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) p[u] = __builtin_amdgcn_exp2f(lg[u][g] - mnew);
        st.l[g] = fmaf(st.l[g], sc, (p[0] + p[1]) + (p[2] + p[3]));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float t = st.acc[g][e] * sc;
            t = fmaf(p[0], x[0][e], t);
            t = fmaf(p[1], x[1][e], t);
            t = fmaf(p[2], x[2][e], t);
            t = fmaf(p[3], x[3][e], t);
            st.acc[g][e] = t;
        }
        st.m[g] = mnew;
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

// Dot products of 4 rows with the G scaled queries (logits in base-2 units).
template <typename T, int G>
__device__ __forceinline__ void logits4(const float (&qs)[G][8], const Slice8<T> (&k)[4], const bool (&valid)[4],
                                        float (&lg)[4][G]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        float x[8];
        k[u].unpack(x);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float d = qs[g][0] * x[0];
#pragma unroll
            for (int e = 1; e < 8; ++e) d = fmaf(qs[g][e], x[e], d);
            d = row16_sum(d);
            lg[u][g] = valid[u] ? d : -INFINITY;
        }
    }
}

// Row buffers of one step: 4 rows per row group (row i = step*64 + wave*16 +
// u*4 + rg of the staged list).
template <typename T>
struct RowBuf {
    Slice8<T> k[4], v[4];
    bool ok[4];
};
template <typename T>
struct PseudoBuf {
    Slice8<T> v[4];
    bool ok[4];
    int i[4];
};

template <typename T>
__device__ __forceinline__ void load_rows(RowBuf<T>& bf, const int32_t* s_row, int cnt, int it, int wave, int rg,
                                          const T* Kx, const T* Vx) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = it * 64 + wave * 16 + u * 4 + rg;
        bf.ok[u] = i < cnt;
        const int r = s_row[bf.ok[u] ? i : 0];
        bf.k[u].load(Kx + (size_t)r * kHeadDim);
        bf.v[u].load(Vx + (size_t)r * kHeadDim);
    }
}

template <typename T, int G>
__device__ __forceinline__ void exact_step(SoftState<G>& st, const float (&qs)[G][8], const RowBuf<T>& bf) {
    float lg[4][G];
    logits4<T, G>(qs, bf.k, bf.ok, lg);
    absorb4<T, G>(st, lg, bf.v);
}

template <typename T>
__device__ __forceinline__ void load_pseudo(PseudoBuf<T>& bf, const int32_t* s_pid, int cnt, int it, int wave, int rg,
                                            const T* vbar) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int i = it * 64 + wave * 16 + u * 4 + rg;
        bf.ok[u] = i < cnt;
        bf.i[u] = bf.ok[u] ? i : 0;
        bf.v[u].load(vbar + (size_t)s_pid[bf.i[u]] * kHeadDim);
    }
}

template <typename T, int G>
__device__ __forceinline__ void pseudo_step(SoftState<G>& st, const float (*s_plg)[G], const PseudoBuf<T>& bf) {
    float lg[4][G];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int g = 0; g < G; ++g) lg[u][g] = bf.ok[u] ? s_plg[bf.i[u]][g] : -INFINITY;
    absorb4<T, G>(st, lg, bf.v);
}

template <typename T, int G>
__global__ __launch_bounds__(256) void attend_kernel(AttendArgs a) {
    __shared__ int32_t s_row[kAttCap];
    __shared__ int32_t s_pid[kAttCap];
    __shared__ float s_plg[kAttCap][G];
    __shared__ float s_red[4][G][kHeadDim + 2];

    const int split = blockIdx.x, unit = blockIdx.y;
    const int S = a.S;
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int b = unit / a.Hkv, h = unit % a.Hkv;

    const T* qb = reinterpret_cast<const T*>(a.q) + ((size_t)b * a.Hq + (size_t)h * G) * kHeadDim + li * 8;
    float qs[G][8];
    const float qscale = kInvSqrtD * kLog2e;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Slice8<T> s;
        s.load(qb + (size_t)g * kHeadDim);
        s.unpack(qs[g]);
#pragma unroll
        for (int e = 0; e < 8; ++e) qs[g][e] *= qscale;
    }
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

    // ---- exact rows of selected clusters -------------------------------
    {
        const int E = a.row_counts[unit * 4];
        const int e0 = (int)((int64_t)E * split / S), e1 = (int)((int64_t)E * (split + 1) / S);
        const int32_t* rws = a.rows + (size_t)unit * a.row_stride;
        const int32_t* tids = a.token_ids ? a.token_ids + (size_t)unit * a.Nmax : nullptr;
        for (int c0 = e0; c0 < e1; c0 += kAttCap) {
            const int cnt = min(kAttCap, e1 - c0);
            __syncthreads();
            for (int i = tid; i < cnt; i += 256) {
                const int pos = rws[c0 + i];
                s_row[i] = tids ? tids[pos] : pos;
            }
            __syncthreads();
            const int steps = (cnt + 63) / 64;
            RowBuf<T> A, B;
            if (steps > 0) load_rows<T>(A, s_row, cnt, 0, wave, rg, Kx, Vx);
            for (int it = 0; it < steps; it += 2) {
                if (it + 1 < steps) load_rows<T>(B, s_row, cnt, it + 1, wave, rg, Kx, Vx);
                exact_step<T, G>(st, qs, A);
                if (it + 1 < steps) {
                    if (it + 2 < steps) load_rows<T>(A, s_row, cnt, it + 2, wave, rg, Kx, Vx);
                    exact_step<T, G>(st, qs, B);
                }
            }
        }
    }
    // ---- unclustered tail, attended exactly ------------------------------
    {
        const int Tn = a.n_total - a.n_clustered;
        const int t0 = (int)((int64_t)Tn * split / S), t1 = (int)((int64_t)Tn * (split + 1) / S);
        const T* Kt = reinterpret_cast<const T*>(a.K) + ubase;
        const T* Vt = reinterpret_cast<const T*>(a.V) + ubase;
        for (int base = t0 + wave * 16; base < t1; base += 64) {
            Slice8<T> kb[4], vb[4];
            bool ok[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = base + u * 4 + rg;
                ok[u] = i < t1;
                const int r = a.n_clustered + (ok[u] ? i : t0);
                kb[u].load(Kt + (size_t)r * kHeadDim);
                vb[u].load(Vt + (size_t)r * kHeadDim);
            }
            float lg[4][G];
            logits4<T, G>(qs, kb, ok, lg);
            absorb4<T, G>(st, lg, vb);
        }
    }
    // ---- approximated clusters: logit s + ln n, value Vbar ----------------
#pragma unroll 1
    for (int which = 0; which < 2; ++which) {
        const PseudoList& pl = which == 0 ? a.pa : a.pb;
        if (!pl.list) continue;
        const int P = pl.counts[unit * 4 + 1];
        const int p0 = (int)((int64_t)P * split / S), p1 = (int)((int64_t)P * (split + 1) / S);
        const int32_t* lst = pl.list + (size_t)unit * pl.stride;
        const float* su = pl.s + (size_t)unit * pl.rows * G;
        const int32_t* szu = pl.sizes + (size_t)unit * pl.rows;
        const T* vbar = reinterpret_cast<const T*>(pl.vbar) + (size_t)unit * pl.rows * kHeadDim + li * 8;
        for (int c0 = p0; c0 < p1; c0 += kAttCap) {
            const int cnt = min(kAttCap, p1 - c0);
            __syncthreads();
            for (int i = tid; i < cnt; i += 256) {
                const int c = lst[c0 + i];
                s_pid[i] = c;
                const float ln2n = __builtin_amdgcn_logf((float)szu[c]);  // log2(n)
#pragma unroll
                for (int g = 0; g < G; ++g) s_plg[i][g] = fmaf(su[(size_t)c * G + g], kLog2e, ln2n);
            }
            __syncthreads();
            const int steps = (cnt + 63) / 64;
            PseudoBuf<T> A, B;
            if (steps > 0) load_pseudo<T>(A, s_pid, cnt, 0, wave, rg, vbar);
            for (int it = 0; it < steps; it += 2) {
                if (it + 1 < steps) load_pseudo<T>(B, s_pid, cnt, it + 1, wave, rg, vbar);
                pseudo_step<T, G>(st, s_plg, A);
                if (it + 1 < steps) {
                    if (it + 2 < steps) load_pseudo<T>(A, s_pid, cnt, it + 2, wave, rg, vbar);
                    pseudo_step<T, G>(st, s_plg, B);
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
    hipLaunchKernelGGL(select_kernel, dim3(units), dim3(64), 0, st, a);
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
