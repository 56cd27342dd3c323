// kmeans.hip -- blockwise k-means of the key cache on gfx950.
//
// Keys of each (sequence, KV head) unit are grouped by k-means inside blocks
// of the sequence, one centroid per `tpc` tokens (mlsanity.com paper page,
// "Abstract (arXiv)": keys clustered by semantic similarity; atlas.scime.ai
// summary, "Approach": blockwise clustering; "Measured effects reported in the
// paper": one centroid per 16 tokens and blocks of a few thousand tokens).
//
// One Lloyd round is three launches:
//   assign  -- keys x centroids contraction on bf16 MFMA (fp32 accumulate);
//              the nearest centroid is the argmax of k.mu - |mu|^2 / 2, folded
//              into the accumulator initial value, ties to the lowest id;
//   csr     -- per block, the membership lists in (cluster, token) order,
//              sizes and offsets: a stable counting sort in LDS for blocks of
//              up to 1024 clusters, an LDS bitonic sort of (cluster, token)
//              keys beyond (the same result, deterministic);
//   mean    -- segmented mean of member rows, fixed summation order.
#include <math.h>

#include <type_traits>

#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__device__ __forceinline__ void block_info(const BlockRange& br, int j, int& p, int& L, int& c0, int& C) {
    p = br.p_base + j * br.block_len;
    L = min(br.block_len, br.n_end - p);
    c0 = br.c_base + j * br.cfull;
    C = (L + br.tpc - 1) / br.tpc;
}

// ---------------------------------------------------------------------------
// Seeded initialisation: C distinct tokens of the block, the first C steps of
// a Fisher-Yates shuffle driven by splitmix64 used as a counter-based
// generator (draw t = mix(s0 + (t + 1) * gamma), s0 = seed ^ mix(unit << 32 |
// block)).  Draws are computed in parallel; the C swaps run in one lane.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void kmeans_init_kernel(const T* __restrict__ K, UnitGeom g, BlockRange br,
                                                          uint64_t seed, float* __restrict__ mu,
                                                          T* __restrict__ kbar) {
    __shared__ uint16_t perm[kMaxBlock];
    __shared__ uint16_t pick[kMaxBlock];
    const int j = blockIdx.x, unit = blockIdx.y;
    int p, L, c0, C;
    block_info(br, j, p, L, c0, C);
    for (int i = threadIdx.x; i < L; i += blockDim.x) perm[i] = (uint16_t)i;
    const uint64_t s0 = seed ^ sm64_mix(((uint64_t)unit << 32) + (uint64_t)(br.j_base + j));
    for (int t = threadIdx.x; t < C; t += blockDim.x) {
        const uint64_t x = sm64_mix(s0 + (uint64_t)(t + 1) * kSm64Gamma);
        pick[t] = (uint16_t)(t + (int)(x % (uint64_t)(L - t)));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int t = 0; t < C; ++t) {
            const int r = pick[t];
            const uint16_t a = perm[t];
            perm[t] = perm[r];
            perm[r] = a;
        }
    }
    __syncthreads();
    const T* Ku = K + (size_t)unit * g.Nmax * kHeadDim;
    const size_t cbase = (size_t)unit * g.Cmax * kHeadDim;
    for (int e = threadIdx.x; e < C * 16; e += blockDim.x) {
        const int c = e >> 4, part = e & 15;
        Slice8<T> s;
        s.load(Ku + (size_t)(p + perm[c]) * kHeadDim + part * 8);
        float x[8];
        s.unpack(x);
        const size_t dst = cbase + (size_t)(c0 + c) * kHeadDim + part * 8;
        store8(mu + dst, x);
        s.store(kbar + dst);
    }
}

// ---------------------------------------------------------------------------
// Assignment, bf16: one workgroup = 64 kAsgWaves tokens of one block (64 per
// wave).  MFMA 32x32x16 with A = 32 centroids (from LDS), B = 32 tokens
// (registers); lane l holds token l % 32 and 16 centroid rows of the tile, so
// the running argmax needs no cross-lane traffic until the end.  The
// accumulator starts at -|mu|^2 / 2 (kept negated in LDS) so the MFMA result
// is the score itself.
// ---------------------------------------------------------------------------
constexpr int kAsgWaves = 4;                     // waves per workgroup
constexpr int kAsgThreads = kAsgWaves * kWave;
constexpr int kAsgTokens = kAsgThreads;          // tokens per workgroup
constexpr int kAsgChunk = 64;                    // centroids staged per LDS round
constexpr int kAsgTiles = kAsgChunk / 32;        // centroid tiles per chunk
constexpr int kAsgStage = kAsgChunk * 16 / kAsgThreads;  // 16-byte parts each thread stages
constexpr int kAsgPad = 17;    // uint4 per staged row (16 + 1 to spread LDS banks)
static_assert(kAsgChunk % 32 == 0 && (kAsgChunk * 16) % kAsgThreads == 0, "chunk staging");

__global__ __launch_bounds__(kAsgThreads) void kmeans_assign_bf16_kernel(const bf16_t* __restrict__ K, UnitGeom g,
                                                                         BlockRange br,
                                                                         const bf16_t* __restrict__ kbar,
                                                                         int32_t* __restrict__ assign, int tiles) {
    // two LDS buffers of staged centroids: chunk ch + 1 is loaded into
    // registers while chunk ch is on the matrix cores, then written to the
    // other buffer (one barrier per chunk)
    __shared__ uint4 cs[2][kAsgChunk * kAsgPad];
    __shared__ __align__(16) float hn[2][kAsgChunk];
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int group = lid / tiles, tile = lid % tiles;
    if (group >= g.units * br.nb) return;
    const int unit = group / br.nb, j = group % br.nb;
    int p, L, c0, C;
    block_info(br, j, p, L, c0, C);
    const int t0 = tile * kAsgTokens;
    if (t0 >= L) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int half = lane >> 5, col = lane & 31;

    const bf16_t* Ku = K + (size_t)unit * g.Nmax * kHeadDim;
    uint4 kb[2][8];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const int tok = t0 + wave * 64 + tb * 32 + col;
        const uint4* row = reinterpret_cast<const uint4*>(Ku + (size_t)(p + min(tok, L - 1)) * kHeadDim);
#pragma unroll
        for (int s = 0; s < 8; ++s) kb[tb][s] = tok < L ? row[2 * s + half] : make_uint4(0, 0, 0, 0);
    }
    float best[2] = {-INFINITY, -INFINITY};
    int bidx[2] = {0x7fffffff, 0x7fffffff};
    const bf16_t* Cu = kbar + ((size_t)unit * g.Cmax + c0) * kHeadDim;

    // thread t stages parts t + T m (m < kAsgStage, T threads) of a chunk:
    // row (t + T m) / 16
    auto fetch = [&](int ch, uint4 (&v)[kAsgStage]) {
#pragma unroll
        for (int m = 0; m < kAsgStage; ++m) {
            const int e = threadIdx.x + m * kAsgThreads;
            const int c = ch + (e >> 4);
            v[m] = c < C ? reinterpret_cast<const uint4*>(Cu + (size_t)c * kHeadDim)[e & 15] : make_uint4(0, 0, 0, 0);
        }
    };
    auto stage = [&](int ch, const uint4 (&v)[kAsgStage], int buf) {
#pragma unroll
        for (int m = 0; m < kAsgStage; ++m) {
            const int e = threadIdx.x + m * kAsgThreads;
            const int row = e >> 4, part = e & 15;
            const int c = ch + row;
            cs[buf][row * kAsgPad + part] = v[m];
            const float x0 = bf16_lo(v[m].x), x1 = bf16_hi(v[m].x), x2 = bf16_lo(v[m].y), x3 = bf16_hi(v[m].y);
            const float x4 = bf16_lo(v[m].z), x5 = bf16_hi(v[m].z), x6 = bf16_lo(v[m].w), x7 = bf16_hi(v[m].w);
            float ss = x0 * x0;
            ss = fmaf(x1, x1, ss); ss = fmaf(x2, x2, ss); ss = fmaf(x3, x3, ss);
            ss = fmaf(x4, x4, ss); ss = fmaf(x5, x5, ss); ss = fmaf(x6, x6, ss); ss = fmaf(x7, x7, ss);
            ss = row16_sum(ss);  // the 16 lanes of a row hold its 16 parts
            if (part == 0) hn[buf][row] = c < C ? -0.5f * ss : -INFINITY;
        }
    };
    {
        uint4 v[kAsgStage];
        fetch(0, v);
        stage(0, v, 0);
    }
    __syncthreads();
    int buf = 0;
    for (int ch = 0; ch < C; ch += kAsgChunk) {
        const bool more = ch + kAsgChunk < C;  // (uniform)
        uint4 nv[kAsgStage];
        if (more) fetch(ch + kAsgChunk, nv);
        // accumulators start at -|mu|^2 / 2 of their centroid rows (the
        // first product takes them as its addend)
        f32x16_t init[kAsgTiles];
#pragma unroll
        for (int cb = 0; cb < kAsgTiles; ++cb)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) {
                const float4 h = *reinterpret_cast<const float4*>(&hn[buf][cb * 32 + 8 * q4 + 4 * half]);
                init[cb][4 * q4 + 0] = h.x;
                init[cb][4 * q4 + 1] = h.y;
                init[cb][4 * q4 + 2] = h.z;
                init[cb][4 * q4 + 3] = h.w;
            }
        f32x16_t acc[kAsgTiles][2];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int cb = 0; cb < kAsgTiles; ++cb) {
                const uint4 a = cs[buf][(cb * 32 + col) * kAsgPad + 2 * s + half];
                const bf16x8_t av = __builtin_bit_cast(bf16x8_t, a);
#pragma unroll
                for (int tb = 0; tb < 2; ++tb)
                    acc[cb][tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        av, __builtin_bit_cast(bf16x8_t, kb[tb][s]), s == 0 ? init[cb] : acc[cb][tb], 0, 0, 0);
            }
        }
        // the rows this lane holds increase with the register index, and
        // tiles are visited in increasing id order: a tile replaces the
        // running best only when its maximum is strictly larger, taking the
        // lowest row that reaches it (ties keep the lowest id).  The maximum
        // takes 8 three-way max instructions; the row search runs only in
        // waves where some lane improved.
#pragma unroll
        for (int cb = 0; cb < kAsgTiles; ++cb)
#pragma unroll
            for (int tb = 0; tb < 2; ++tb) {
                const f32x16_t v = acc[cb][tb];
                float m = fmaxf(fmaxf(v[0], v[1]), v[2]);
                m = fmaxf(fmaxf(m, v[3]), v[4]);
                m = fmaxf(fmaxf(m, v[5]), v[6]);
                m = fmaxf(fmaxf(m, v[7]), v[8]);
                m = fmaxf(fmaxf(m, v[9]), v[10]);
                m = fmaxf(fmaxf(m, v[11]), v[12]);
                m = fmaxf(fmaxf(m, v[13]), v[14]);
                m = fmaxf(m, v[15]);
                if (m > best[tb]) {
                    int r = 15;
#pragma unroll
                    for (int k = 14; k >= 0; --k) r = v[k] == m ? k : r;
                    best[tb] = m;
                    bidx[tb] = ch + cb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                }
            }
        if (more) stage(ch + kAsgChunk, nv, buf ^ 1);  // the other buffer: read by no wave now
        __syncthreads();
        buf ^= 1;
    }
    int32_t* au = assign + (size_t)unit * g.Nmax + p;
#pragma unroll
    for (int tb = 0; tb < 2; ++tb) {
        const float ov = shfl_xor_f(best[tb], 32);
        const int oi = shfl_xor_i(bidx[tb], 32);
        if (ov > best[tb] || (ov == best[tb] && oi < bidx[tb])) bidx[tb] = oi;
        const int tok = t0 + wave * 64 + tb * 32 + col;
        if (half == 0 && tok < L) au[tok] = c0 + bidx[tb];
    }
}

// Assignment, fp32 storage: one thread per token, FMA dot products against
// 32 centroids staged in LDS at a time; same score and tie rule.
__global__ __launch_bounds__(256) void kmeans_assign_f32_kernel(const float* __restrict__ K, UnitGeom g,
                                                                BlockRange br, const float* __restrict__ kbar,
                                                                int32_t* __restrict__ assign, int tiles) {
    __shared__ float cs[32][kHeadDim];
    __shared__ float hn[32];
    const int lid = xcd_logical_id(blockIdx.x, gridDim.x);
    const int group = lid / tiles, tile = lid % tiles;
    if (group >= g.units * br.nb) return;
    const int unit = group / br.nb, j = group % br.nb;
    int p, L, c0, C;
    block_info(br, j, p, L, c0, C);
    const int t0 = tile * 256;
    if (t0 >= L) return;
    const int tok = t0 + threadIdx.x;
    const bool valid = tok < L;
    float k[kHeadDim];
    const float* krow = K + ((size_t)unit * g.Nmax + p + min(tok, L - 1)) * kHeadDim;
#pragma unroll
    for (int e = 0; e < kHeadDim; e += 4) {
        const float4 v = *reinterpret_cast<const float4*>(krow + e);
        k[e] = v.x; k[e + 1] = v.y; k[e + 2] = v.z; k[e + 3] = v.w;
    }
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    const float* Cu = kbar + ((size_t)unit * g.Cmax + c0) * kHeadDim;
    for (int ch = 0; ch < C; ch += 32) {
        for (int e = threadIdx.x; e < 32 * kHeadDim; e += 256) {
            const int row = e / kHeadDim, cc = e % kHeadDim;
            cs[row][cc] = ch + row < C ? Cu[(size_t)(ch + row) * kHeadDim + cc] : 0.f;
        }
        __syncthreads();
        if (threadIdx.x < 32) {
            float ss = 0.f;
            for (int e = 0; e < kHeadDim; ++e) ss = fmaf(cs[threadIdx.x][e], cs[threadIdx.x][e], ss);
            hn[threadIdx.x] = ch + (int)threadIdx.x < C ? 0.5f * ss : INFINITY;
        }
        __syncthreads();
        for (int r = 0; r < 32; ++r) {
            float v = -hn[r];
#pragma unroll
            for (int e = 0; e < kHeadDim; ++e) v = fmaf(k[e], cs[r][e], v);
            if (v > best) {
                best = v;
                bidx = ch + r;
            }
        }
        __syncthreads();
    }
    if (valid) assign[(size_t)unit * g.Nmax + p + tok] = c0 + bidx;
}

// ---------------------------------------------------------------------------
// Membership lists: per block, sort the keys (local cluster << 14 | local
// token) with a bitonic network in LDS.  The sorted order is (cluster, token),
// which fixes token_ids; offsets are lower bounds of each cluster id.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int lds_lower_bound(const uint32_t* a, int n, uint32_t key) {
    int lo = 0, hi = n;
    while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (a[mid] < key) lo = mid + 1;
        else hi = mid;
    }
    return lo;
}

constexpr int kCsrThreads = 1024;

// A bitonic sort of P2 = K * kCsrThreads keys, thread t holding keys
// t K .. t K + K - 1 in v: exchanges at distance jj < K stay in the thread,
// jj < 64 K cross lanes of a wave (shuffles), larger ones go through LDS
// (`keys`).  Sorted, the keys are back in `keys`.
template <int K>
__device__ __forceinline__ void csr_sort(uint32_t* keys, const int32_t* au, int L, int c0) {
    constexpr int P2 = K * kCsrThreads;
    const int t = threadIdx.x;
    uint32_t v[K];
#pragma unroll
    for (int q = 0; q < K; ++q) {
        const int i = t * K + q;
        v[q] = i < L ? ((uint32_t)(au[i] - c0) << 14) | (uint32_t)i : 0xFFFFFFFFu;
    }
    for (int k = 2; k <= P2; k <<= 1) {
        for (int jj = k >> 1; jj > 0; jj >>= 1) {
            if (jj >= kWave * K) {  // (uniform) partner in another wave
#pragma unroll
                for (int q = 0; q < K; ++q) keys[t * K + q] = v[q];
                __syncthreads();
#pragma unroll
                for (int q = 0; q < K; ++q) {
                    const int i = t * K + q;
                    const uint32_t b = keys[i ^ jj];
                    const bool keep_min = ((i & jj) == 0) == ((i & k) == 0);
                    v[q] = keep_min ? min(v[q], b) : max(v[q], b);
                }
                __syncthreads();  // before the keys are written again
            } else if (jj >= K) {  // (uniform) partner in another lane of the wave
                const int lj = jj / K;
                uint32_t b[K];
#pragma unroll
                for (int q = 0; q < K; ++q) b[q] = (uint32_t)__shfl_xor((int)v[q], lj, kWave);
#pragma unroll
                for (int q = 0; q < K; ++q) {
                    const int i = t * K + q;
                    const bool keep_min = ((i & jj) == 0) == ((i & k) == 0);
                    v[q] = keep_min ? min(v[q], b[q]) : max(v[q], b[q]);
                }
            } else {  // partner in the same thread
#pragma unroll
                for (int q = 0; q < K; ++q) {
                    if ((q & jj) == 0) {
                        const int i = t * K + q;
                        const uint32_t a = v[q], b = v[q ^ jj];
                        const bool asc = (i & k) == 0;
                        v[q] = asc ? min(a, b) : max(a, b);
                        v[q ^ jj] = asc ? max(a, b) : min(a, b);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < K; ++q) keys[t * K + q] = v[q];
    __syncthreads();
}

__global__ __launch_bounds__(kCsrThreads) void kmeans_csr_kernel(const int32_t* __restrict__ assign, UnitGeom g,
                                                                 BlockRange br, int32_t* __restrict__ sizes,
                                                                 int32_t* __restrict__ offsets,
                                                                 int32_t* __restrict__ token_ids) {
    __shared__ uint32_t keys[kMaxBlock];
    const int j = blockIdx.x, unit = blockIdx.y;
    int p, L, c0, C;
    block_info(br, j, p, L, c0, C);
    // keys cluster << 14 | token, sorted (distinct keys: the (cluster, token)
    // order); the keys past L sort last
    int P2 = kCsrThreads;
    while (P2 < L) P2 <<= 1;
    const int32_t* au = assign + (size_t)unit * g.Nmax + p;
    switch (P2 / kCsrThreads) {  // (uniform)
        case 1: csr_sort<1>(keys, au, L, c0); break;
        case 2: csr_sort<2>(keys, au, L, c0); break;
        case 4: csr_sort<4>(keys, au, L, c0); break;
        case 8: csr_sort<8>(keys, au, L, c0); break;
        default: csr_sort<16>(keys, au, L, c0); break;
    }
    int32_t* tu = token_ids + (size_t)unit * g.Nmax;
    for (int pos = threadIdx.x; pos < L; pos += blockDim.x) tu[p + pos] = p + (int)(keys[pos] & 0x3FFFu);
    int32_t* su = sizes + (size_t)unit * g.Cmax;
    int32_t* ou = offsets + (size_t)unit * (g.Cmax + 1);
    for (int c = threadIdx.x; c < C; c += blockDim.x) {
        const int lo = lds_lower_bound(keys, L, (uint32_t)c << 14);
        const int hi = lds_lower_bound(keys, L, (uint32_t)(c + 1) << 14);
        ou[c0 + c] = p + lo;
        su[c0 + c] = hi - lo;
    }
    if (threadIdx.x == 0) ou[c0 + C] = p + L;
}


// Membership lists by a stable counting sort, for blocks of at most
// kCountMaxC clusters: the same (cluster, token) order, sizes and offsets as
// the sort above, in three LDS passes.  Wave w owns tokens [w R 64, (w + 1)
// R 64) of the block (R rounds of 64); it counts its tokens per cluster;
// per cluster the counts are turned into bases (clusters in order, then
// waves in order); then each wave places its rounds in order.  Inside a
// round the 64 (cluster, lane) keys are sorted across the lanes (a bitonic
// network over lane shuffles), so the lanes of one cluster are placed in
// lane, that is token, order: rank = sorted position - first position of the
// cluster, and the cluster's last lane moves its base on.
constexpr int kCountMaxC = 1024;

// Inclusive maximum over the 64 lanes of non-negative values (DPP as in
// wave_inclusive_sum; lanes without a source take 0).
__device__ __forceinline__ int wave_inclusive_max(int v) {
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false));  // row_shr:1
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false));  // row_shr:2
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false));  // row_shr:4
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false));  // row_shr:8
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false));  // row_bcast:15 -> rows 1, 3
    v = max(v, __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false));  // row_bcast:31 -> rows 2, 3
    return v;
}

__global__ __launch_bounds__(kCsrThreads) void kmeans_csr_count_kernel(const int32_t* __restrict__ assign,
                                                                       UnitGeom g, BlockRange br,
                                                                       int32_t* __restrict__ sizes,
                                                                       int32_t* __restrict__ offsets,
                                                                       int32_t* __restrict__ token_ids) {
    constexpr int kWaves = kCsrThreads / kWave;
    __shared__ uint32_t base[kWaves][kCountMaxC];  // counts, then bases
    __shared__ int32_t placed[kMaxBlock];          // token ids in member order
    __shared__ int wsum[kWaves];
    const int j = blockIdx.x, unit = blockIdx.y;
    int p, L, c0, C;
    block_info(br, j, p, L, c0, C);
    const int tid = threadIdx.x, wave = tid / kWave, lane = tid & (kWave - 1);
    const int rounds = (L + kCsrThreads - 1) / kCsrThreads;
    const int w0 = wave * kWave * rounds;  // the wave's first token
    const int32_t* au = assign + (size_t)unit * g.Nmax + p;
    // a token's local cluster; an id outside the block (no finite score won
    // its argmax) counts as the last cluster, so every token is placed once
    auto local = [&](int i) { return min((uint32_t)(au[i] - c0), (uint32_t)(C - 1)); };
    for (int e = tid; e < kWaves * kCountMaxC; e += kCsrThreads) (&base[0][0])[e] = 0u;
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        const int i = w0 + r * kWave + lane;
        if (i < L) atomicAdd(&base[wave][local(i)], 1u);
    }
    __syncthreads();
    // cluster tid: bases over the waves, then over the clusters
    int total = 0;
    if (tid < C) {
        for (int w = 0; w < kWaves; ++w) {
            const uint32_t t = base[w][tid];
            base[w][tid] = (uint32_t)total;
            total += (int)t;
        }
    }
    const int inc = wave_inclusive_sum(total);
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    int off = inc - total;
    for (int w = 0; w < wave; ++w) off += wsum[w];
    int32_t* su = sizes + (size_t)unit * g.Cmax;
    int32_t* ou = offsets + (size_t)unit * (g.Cmax + 1);
    if (tid < C) {
        for (int w = 0; w < kWaves; ++w) base[w][tid] += (uint32_t)off;
        ou[c0 + tid] = p + off;
        su[c0 + tid] = total;
    }
    if (tid == 0) ou[c0 + C] = p + L;
    __syncthreads();
    for (int r = 0; r < rounds; ++r) {
        const int i = w0 + r * kWave + lane;
        uint32_t key = i < L ? (local(i) << 6) | (uint32_t)lane : 0xFFFFFFFFu;
#pragma unroll
        for (int k = 2; k <= kWave; k <<= 1)
#pragma unroll
            for (int jj = k >> 1; jj > 0; jj >>= 1) {
                const uint32_t o = (uint32_t)__shfl_xor((int)key, jj, kWave);
                const bool lower = ((lane & k) == 0) == ((lane & jj) == 0);
                key = lower ? min(key, o) : max(key, o);
            }
        // keys past L (all ones) sort last and are not placed
        const uint32_t c = key >> 6;
        const uint32_t prev = (uint32_t)__shfl_up((int)key, 1, kWave);
        const uint32_t next = (uint32_t)__shfl_down((int)key, 1, kWave);
        const bool first = lane == 0 || (prev >> 6) != c;
        const bool last = lane == kWave - 1 || (next >> 6) != c;
        const int rank = lane - wave_inclusive_max(first ? lane : 0);
        if (key != 0xFFFFFFFFu) {
            const uint32_t b = base[wave][c];
            placed[b + rank] = p + w0 + r * kWave + (int)(key & 63u);
            if (last) base[wave][c] = b + (uint32_t)rank + 1u;
        }
    }
    __syncthreads();
    int32_t* tu = token_ids + (size_t)unit * g.Nmax;
    for (int pos = tid; pos < L; pos += kCsrThreads) tu[p + pos] = placed[pos];
}

// ---------------------------------------------------------------------------
// Segmented mean: one wave per cluster, 16 lanes per row (8 elements each),
// the 4 row groups of the wave take rows g, g + 4, ... in order and are
// combined as (g0 + g1) + (g2 + g3): a fixed order, so results repeat bitwise.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void segmented_mean_kernel(const T* __restrict__ X, UnitGeom g, int c_begin,
                                                             int c_count, const int32_t* __restrict__ sizes,
                                                             const int32_t* __restrict__ offsets,
                                                             const int32_t* __restrict__ token_ids,
                                                             float* __restrict__ master, T* __restrict__ store,
                                                             int empty_zero) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int unit = blockIdx.y;
    const int c = c_begin + blockIdx.x * 4 + wave;
    if (c >= c_begin + c_count) return;
    const int n = sizes[(size_t)unit * g.Cmax + c];
    const size_t crow = ((size_t)unit * g.Cmax + c) * kHeadDim + li * 8;
    if (n == 0) {
        if (empty_zero && rg == 0) {
            const float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
            store8(store + crow, z);
        }
        return;
    }
    const int start = offsets[(size_t)unit * (g.Cmax + 1) + c];
    const int32_t* ids = token_ids + (size_t)unit * g.Nmax + start;
    const T* Xu = X + (size_t)unit * g.Nmax * kHeadDim + li * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    int r = rg;
    for (; r + 4 < n; r += 8) {
        const int ta = ids[r], tb = ids[r + 4];
        Slice8<T> a, b;
        a.load(Xu + (size_t)ta * kHeadDim);
        b.load(Xu + (size_t)tb * kHeadDim);
        float xa[8], xb[8];
        a.unpack(xa);
        b.unpack(xb);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += xa[e];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += xb[e];
    }
    if (r < n) {
        Slice8<T> a;
        a.load(Xu + (size_t)ids[r] * kHeadDim);
        float xa[8];
        a.unpack(xa);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += xa[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += shfl_xor_f(acc[e], 16);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += shfl_xor_f(acc[e], 32);
    if (rg == 0) {
        float m[8];
        const float fn = (float)n;
#pragma unroll
        for (int e = 0; e < 8; ++e) m[e] = acc[e] / fn;
        if (master) store8(master + crow, m);
        store8(store + crow, m);
    }
}

// Cluster-ordered copy of K and V rows (16 lanes per row).
template <typename T>
__global__ __launch_bounds__(256) void sorted_copy_kernel(const T* __restrict__ K, const T* __restrict__ V,
                                                          UnitGeom g, int p_begin, int count,
                                                          const int32_t* __restrict__ token_ids,
                                                          T* __restrict__ SK, T* __restrict__ SV) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int rg = lane >> 4, li = lane & 15;
    const int unit = blockIdx.y;
    const int pos = p_begin + blockIdx.x * 16 + wave * 4 + rg;
    if (pos >= p_begin + count) return;
    const int tok = token_ids[(size_t)unit * g.Nmax + pos];
    const size_t src = ((size_t)unit * g.Nmax + tok) * kHeadDim + li * 8;
    const size_t dst = ((size_t)unit * g.Nmax + pos) * kHeadDim + li * 8;
    Slice8<T> a, b;
    a.load(K + src);
    b.load(V + src);
    a.store(SK + dst);
    b.store(SV + dst);
}

// ---------------------------------------------------------------------------
// Coarse level of the hierarchy, one workgroup per (unit, fine block):
// size-weighted Lloyd k-means over the block's non-empty fine key centroids
// (weights = fine sizes), seeded like the token level with stream level 1;
// then parents, member lists by (coarse, fine), sizes and value centroids
// (size-weighted means of the stored fine value centroids).  With bf16
// storage the assignment runs on the matrix cores (32-point tiles against
// the stored centroids, as the token level does); the weighted means take
// one 16-lane row group per coarse cluster, members in point order.
// ---------------------------------------------------------------------------
constexpr int kCoarseMaxFine = 2048;  // fine clusters per block
constexpr int kCoarseMaxD = 64;       // coarse clusters per block

template <typename T>
__global__ __launch_bounds__(256) void coarse_build_kernel(UnitGeom g, CoarseRange cr, uint64_t seed, int iters,
                                                           const T* __restrict__ kbar, const T* __restrict__ vbar,
                                                           const int32_t* __restrict__ sizes, float* __restrict__ cmu,
                                                           T* __restrict__ ckbar, T* __restrict__ cvbar,
                                                           int32_t* __restrict__ csizes,
                                                           int32_t* __restrict__ parent,
                                                           int32_t* __restrict__ coffsets,
                                                           int32_t* __restrict__ cmembers) {
    __shared__ float cen[kCoarseMaxD][kHeadDim];  // stored (rounded) coarse centroids
    __shared__ float hn[kCoarseMaxD];
    // bf16 storage: the stored centroids as matrix-core operands (rows padded
    // as in the token-level assignment) and their negated half norms (-inf
    // past the D centroids)
    __shared__ uint4 cenb[std::is_same<T, float>::value ? 1 : kCoarseMaxD * kAsgPad];
    __shared__ __align__(16) float hnn[kCoarseMaxD];
    __shared__ int32_t ids[kCoarseMaxFine];       // non-empty fine ids, increasing
    __shared__ int32_t loc[kCoarseMaxFine];       // coarse assignment of each point
    __shared__ uint16_t perm[kCoarseMaxFine];
    __shared__ uint16_t pick[kCoarseMaxD];
    __shared__ uint16_t order[kCoarseMaxFine];    // points by (coarse cluster, point index)
    __shared__ int32_t bstart[kCoarseMaxD + 1];   // start of each coarse cluster in order
    __shared__ float wt[kCoarseMaxFine];          // size of each point (its weight)
    __shared__ int scan_lds[16];
    __shared__ int s_m;
    const int j = blockIdx.x, unit = blockIdx.y;
    int p, L, c0, C;
    block_info(cr.fine, j, p, L, c0, C);
    const int Dfull = (L + cr.coarse_tpc - 1) / cr.coarse_tpc;
    const int g0 = cr.d_base + j * cr.dfull;
    const int32_t* su = sizes + (size_t)unit * g.Cmax;

    // compact the non-empty fine clusters (increasing id)
    int carry = 0;
    for (int base = 0; base < C; base += 256) {
        const int c = base + threadIdx.x;
        const int live = (c < C && su[c0 + c] > 0) ? 1 : 0;
        int4 tot;
        const int4 ex = block256_exclusive_sum4(make_int4(live, 0, 0, 0), tot, scan_lds);
        if (live) ids[carry + ex.x] = c0 + c;
        carry += tot.x;
    }
    // the lists of the blocks follow each other: this block's starts after
    // the non-empty fine clusters of the earlier blocks (of the same build or
    // update alike), so a block's end offset is the next block's start
    int before = 0;
    for (int base = 0; base < c0; base += 256) {
        const int c = base + threadIdx.x;
        int4 tot;
        block256_exclusive_sum4(make_int4(c < c0 && su[c] > 0 ? 1 : 0, 0, 0, 0), tot, scan_lds);
        before += tot.x;
    }
    if (threadIdx.x == 0) s_m = carry;
    __syncthreads();
    const int m = s_m;
    const int D = min(Dfull, m);

    float* cmu_u = cmu + (size_t)unit * cr.Dmax * kHeadDim;
    T* ck_u = ckbar + (size_t)unit * cr.Dmax * kHeadDim;
    T* cv_u = cvbar + (size_t)unit * cr.Dmax * kHeadDim;
    const T* kb_u = kbar + (size_t)unit * g.Cmax * kHeadDim;
    const T* vb_u = vbar + (size_t)unit * g.Cmax * kHeadDim;

    // coarse clusters beyond the non-empty fine count stay empty
    for (int e = threadIdx.x; e < (Dfull - D) * kHeadDim; e += 256) {
        const size_t o = (size_t)(g0 + D) * kHeadDim + e;
        cmu_u[o] = 0.f;
        ck_u[o] = (T)0;
        cv_u[o] = (T)0;
    }
    for (int gg = D + threadIdx.x; gg < Dfull; gg += 256) csizes[(size_t)unit * cr.Dmax + g0 + gg] = 0;

    // seeded init among the m points
    for (int i = threadIdx.x; i < m; i += 256) {
        perm[i] = (uint16_t)i;
        wt[i] = (float)su[ids[i]];
    }
    const uint64_t s0 =
        seed ^ sm64_mix(((uint64_t)unit << 32) + (uint64_t)(cr.fine.j_base + j) + (1ull << 62));
    for (int t = threadIdx.x; t < D; t += 256) {
        const uint64_t x = sm64_mix(s0 + (uint64_t)(t + 1) * kSm64Gamma);
        pick[t] = (uint16_t)(t + (int)(x % (uint64_t)(m - t)));
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int t = 0; t < D; ++t) {
            const int r = pick[t];
            const uint16_t a = perm[t];
            perm[t] = perm[r];
            perm[r] = a;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < D * kHeadDim; e += 256) {
        const int gg = e / kHeadDim, cc = e % kHeadDim;
        const T v = kb_u[(size_t)ids[perm[gg]] * kHeadDim + cc];
        const float f = (float)v;
        cen[gg][cc] = f;
        cmu_u[(size_t)(g0 + gg) * kHeadDim + cc] = f;
    }
    __syncthreads();

    // points of each coarse cluster in increasing point index (a stable
    // counting sort of loc), so the weighted means below visit exactly the
    // members, in point order
    auto bucket = [&]() {
        if (threadIdx.x < D) {
            int n = 0;
            for (int i = 0; i < m; ++i) n += loc[i] == threadIdx.x;
            bstart[threadIdx.x + 1] = n;
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            bstart[0] = 0;
            for (int gg = 0; gg < D; ++gg) bstart[gg + 1] += bstart[gg];
        }
        __syncthreads();
        if (threadIdx.x < D) {
            int k = bstart[threadIdx.x];
            for (int i = 0; i < m; ++i)
                if (loc[i] == threadIdx.x) order[k++] = (uint16_t)i;
        }
        __syncthreads();
    };
    // weighted mean of coarse cluster gg over its members, in point order, by
    // a 16-lane row group: lane li sums columns 8 li .. 8 li + 7 (num), every
    // lane the weights (den; 0 for an empty cluster).  The members' rows load
    // four at a time, so a round trip serves four members.
    const int rgi = threadIdx.x >> 4, li = threadIdx.x & 15;
    constexpr int kGroups = 256 / 16;
    auto wmean8 = [&](const T* src, int gg, float (&num)[8], float& den) {
#pragma unroll
        for (int e = 0; e < 8; ++e) num[e] = 0.f;
        den = 0.f;
        const int k0 = bstart[gg], k1 = bstart[gg + 1];
        for (int kb = k0; kb < k1; kb += 4) {
            float x[4][8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int i = order[min(kb + q, k1 - 1)];
                const T* r = src + (size_t)ids[i] * kHeadDim + li * 8;
#pragma unroll
                for (int e = 0; e < 8; ++e) x[q][e] = (float)r[e];
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (kb + q < k1) {
                    const float w = wt[order[kb + q]];
#pragma unroll
                    for (int e = 0; e < 8; ++e) num[e] = fmaf(w, x[q][e], num[e]);
                    den += w;
                }
            }
        }
    };

    for (int it = 0; it < iters; ++it) {
        if (threadIdx.x < D) {
            float ss = 0.f;
            for (int e = 0; e < kHeadDim; ++e) ss = fmaf(cen[threadIdx.x][e], cen[threadIdx.x][e], ss);
            hn[threadIdx.x] = 0.5f * ss;
        }
        if constexpr (!std::is_same<T, float>::value) {
            // the stored centroids are bf16 values: their bits are the operand
            for (int e = threadIdx.x; e < kCoarseMaxD * 16; e += 256) {
                const int row = e >> 4, part = e & 15;
                uint32_t w[4] = {0u, 0u, 0u, 0u};
                if (row < D) {
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[q] = (__float_as_uint(cen[row][part * 8 + 2 * q]) >> 16) |
                               (__float_as_uint(cen[row][part * 8 + 2 * q + 1]) & 0xFFFF0000u);
                }
                cenb[row * kAsgPad + part] = make_uint4(w[0], w[1], w[2], w[3]);
            }
        }
        __syncthreads();
        if constexpr (!std::is_same<T, float>::value) {
            if (threadIdx.x < kCoarseMaxD) hnn[threadIdx.x] = threadIdx.x < D ? -hn[threadIdx.x] : -INFINITY;
            __syncthreads();
            // assign each point to the best stored centroid (lowest id on
            // ties) on the matrix cores, as the token-level assignment does:
            // 32-point tiles per wave, the accumulator starts at -|mu|^2 / 2
            const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
            const int half = lane >> 5, col = lane & 31;
            for (int t0 = wave * 32; t0 < m; t0 += 4 * 32) {
                const int pt = t0 + col;
                const uint4* row = reinterpret_cast<const uint4*>(kb_u + (size_t)ids[min(pt, m - 1)] * kHeadDim);
                uint4 kr[8];
#pragma unroll
                for (int s = 0; s < 8; ++s) kr[s] = row[2 * s + half];
                f32x16_t acc[2];
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) {
                        const float4 h = *reinterpret_cast<const float4*>(&hnn[cb * 32 + 8 * q4 + 4 * half]);
                        acc[cb][4 * q4 + 0] = h.x;
                        acc[cb][4 * q4 + 1] = h.y;
                        acc[cb][4 * q4 + 2] = h.z;
                        acc[cb][4 * q4 + 3] = h.w;
                    }
#pragma unroll
                for (int s = 0; s < 8; ++s)
#pragma unroll
                    for (int cb = 0; cb < 2; ++cb)
                        acc[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8_t, cenb[(cb * 32 + col) * kAsgPad + 2 * s + half]),
                            __builtin_bit_cast(bf16x8_t, kr[s]), acc[cb], 0, 0, 0);
                // value r of tile cb is centroid cb 32 + 8 (r / 4) + 4 half + r % 4:
                // increasing with (cb, r), so a strict comparison keeps the
                // lowest id among equal maxima
                float best = -INFINITY;
                int bidx = 0x7fffffff;
#pragma unroll
                for (int cb = 0; cb < 2; ++cb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (acc[cb][r] > best) {
                            best = acc[cb][r];
                            bidx = cb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                        }
                const float ov = shfl_xor_f(best, 32);
                const int oi = shfl_xor_i(bidx, 32);
                if (ov > best || (ov == best && oi < bidx)) bidx = oi;
                if (half == 0 && pt < m) loc[pt] = bidx;
            }
        } else {
        // assign each point to the best stored centroid (lowest id on ties);
        // the point's row is held in registers, the centroids are LDS
        // broadcasts
        for (int i = threadIdx.x; i < m; i += 256) {
            const T* x = kb_u + (size_t)ids[i] * kHeadDim;
            float xr[kHeadDim];
#pragma unroll
            for (int e = 0; e < kHeadDim; ++e) xr[e] = (float)x[e];
            float best = -INFINITY;
            int bi = 0;
            for (int gg = 0; gg < D; ++gg) {
                float v = -hn[gg];
#pragma unroll
                for (int e = 0; e < kHeadDim; ++e) v = fmaf(xr[e], cen[gg][e], v);
                if (v > best) {
                    best = v;
                    bi = gg;
                }
            }
            loc[i] = bi;
        }
        }
        __syncthreads();
        bucket();
        // weighted means in point order; empty clusters keep their centroid
        for (int gg = rgi; gg < D; gg += kGroups) {
            float num[8], den;
            wmean8(kb_u, gg, num, den);
            if (den > 0.f) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float mean = num[e] / den;
                    cmu_u[(size_t)(g0 + gg) * kHeadDim + li * 8 + e] = mean;
                    cen[gg][li * 8 + e] = (float)(T)mean;
                }
            }
        }
        __syncthreads();
    }
    // stored coarse key centroids, sizes, value centroids
    for (int gg = rgi; gg < D; gg += kGroups) {
        float num[8], den;
        wmean8(vb_u, gg, num, den);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            ck_u[(size_t)(g0 + gg) * kHeadDim + li * 8 + e] = (T)cen[gg][li * 8 + e];
            cv_u[(size_t)(g0 + gg) * kHeadDim + li * 8 + e] = den > 0.f ? (T)(num[e] / den) : (T)0;
        }
    }
    // parents (-1 for empty fine clusters)
    int32_t* pu = parent + (size_t)unit * g.Cmax;
    for (int c = threadIdx.x; c < C; c += 256) pu[c0 + c] = -1;
    __syncthreads();
    for (int i = threadIdx.x; i < m; i += 256) pu[ids[i]] = g0 + loc[i];
    // member lists by (coarse, fine), one thread for the block
    int32_t* ou = coffsets + (size_t)unit * (cr.Dmax + 1);
    int32_t* mu_ = cmembers + (size_t)unit * g.Cmax;
    for (int gg = threadIdx.x; gg <= Dfull; gg += 256) ou[g0 + gg] = before + (gg < D ? bstart[gg] : m);
    for (int gg = threadIdx.x; gg < D; gg += 256) {
        int tot = 0;
        for (int k = bstart[gg]; k < bstart[gg + 1]; ++k) {
            const int i = order[k];
            mu_[before + k] = ids[i];
            tot += su[ids[i]];
        }
        csizes[(size_t)unit * cr.Dmax + g0 + gg] = tot;
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
static inline int pad_to_xcds(int n) { return (n + kXcds - 1) / kXcds * kXcds; }

hipError_t launch_kmeans_init(int dtype, const void* K, UnitGeom g, BlockRange br, uint64_t seed, float* mu,
                              void* kbar, hipStream_t st) {
    dim3 grid(br.nb, g.units);
    if (dtype == 1)
        hipLaunchKernelGGL(kmeans_init_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)K, g, br, seed, mu,
                           (bf16_t*)kbar);
    else
        hipLaunchKernelGGL(kmeans_init_kernel<float>, grid, dim3(256), 0, st, (const float*)K, g, br, seed, mu,
                           (float*)kbar);
    return hipGetLastError();
}

hipError_t launch_kmeans_assign(int dtype, const void* K, UnitGeom g, BlockRange br, const void* kbar,
                                int32_t* assign, hipStream_t st) {
    const int groups = g.units * br.nb;
    if (dtype == 1) {
        const int tiles = (br.block_len + kAsgTokens - 1) / kAsgTokens;
        const int grid = pad_to_xcds(groups * tiles);
        hipLaunchKernelGGL(kmeans_assign_bf16_kernel, dim3(grid), dim3(kAsgThreads), 0, st, (const bf16_t*)K, g, br,
                           (const bf16_t*)kbar, assign, tiles);
    } else {
        const int tiles = (br.block_len + 255) / 256;
        const int grid = pad_to_xcds(groups * tiles);
        hipLaunchKernelGGL(kmeans_assign_f32_kernel, dim3(grid), dim3(256), 0, st, (const float*)K, g, br,
                           (const float*)kbar, assign, tiles);
    }
    return hipGetLastError();
}

hipError_t launch_kmeans_csr(const int32_t* assign, UnitGeom g, BlockRange br, int32_t* sizes, int32_t* offsets,
                             int32_t* token_ids, hipStream_t st) {
    if (br.cfull <= kCountMaxC)
        hipLaunchKernelGGL(kmeans_csr_count_kernel, dim3(br.nb, g.units), dim3(kCsrThreads), 0, st, assign, g, br,
                           sizes, offsets, token_ids);
    else
        hipLaunchKernelGGL(kmeans_csr_kernel, dim3(br.nb, g.units), dim3(kCsrThreads), 0, st, assign, g, br, sizes,
                           offsets, token_ids);
    return hipGetLastError();
}

hipError_t launch_segmented_mean(int dtype, const void* X, UnitGeom g, int c_begin, int c_count,
                                 const int32_t* sizes, const int32_t* offsets, const int32_t* token_ids,
                                 float* master, void* store, bool empty_zero, hipStream_t st) {
    if (c_count <= 0) return hipSuccess;
    dim3 grid((c_count + 3) / 4, g.units);
    if (dtype == 1)
        hipLaunchKernelGGL(segmented_mean_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)X, g, c_begin,
                           c_count, sizes, offsets, token_ids, master, (bf16_t*)store, (int)empty_zero);
    else
        hipLaunchKernelGGL(segmented_mean_kernel<float>, grid, dim3(256), 0, st, (const float*)X, g, c_begin,
                           c_count, sizes, offsets, token_ids, master, (float*)store, (int)empty_zero);
    return hipGetLastError();
}

hipError_t launch_sorted_copy(int dtype, const void* K, const void* V, UnitGeom g, int p_begin, int count,
                              const int32_t* token_ids, void* SK, void* SV, hipStream_t st) {
    if (count <= 0) return hipSuccess;
    dim3 grid((count + 15) / 16, g.units);
    if (dtype == 1)
        hipLaunchKernelGGL(sorted_copy_kernel<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)K, (const bf16_t*)V, g,
                           p_begin, count, token_ids, (bf16_t*)SK, (bf16_t*)SV);
    else
        hipLaunchKernelGGL(sorted_copy_kernel<float>, grid, dim3(256), 0, st, (const float*)K, (const float*)V, g,
                           p_begin, count, token_ids, (float*)SK, (float*)SV);
    return hipGetLastError();
}

hipError_t launch_coarse_build(int dtype, UnitGeom g, CoarseRange cr, uint64_t seed, int iters, const void* kbar,
                               const void* vbar, const int32_t* sizes, float* cmu, void* ckbar, void* cvbar,
                               int32_t* csizes, int32_t* parent, int32_t* coffsets, int32_t* cmembers,
                               hipStream_t st) {
    dim3 grid(cr.fine.nb, g.units);
    if (dtype == 1)
        hipLaunchKernelGGL(coarse_build_kernel<__bf16>, grid, dim3(256), 0, st, g, cr, seed, iters,
                           (const __bf16*)kbar, (const __bf16*)vbar, sizes, cmu, (__bf16*)ckbar, (__bf16*)cvbar,
                           csizes, parent, coffsets, cmembers);
    else
        hipLaunchKernelGGL(coarse_build_kernel<float>, grid, dim3(256), 0, st, g, cr, seed, iters,
                           (const float*)kbar, (const float*)vbar, sizes, cmu, (float*)ckbar, (float*)cvbar, csizes,
                           parent, coffsets, cmembers);
    return hipGetLastError();
}

}  // namespace mpa
