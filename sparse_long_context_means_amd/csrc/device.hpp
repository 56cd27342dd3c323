// device.hpp -- small device-side helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mpa {

constexpr int kHeadDim = 128;          // the only supported head dimension
constexpr int kWave = 64;              // CDNA wavefront width
constexpr int kXcds = 8;               // accelerator complex dies of an MI355X
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kInvSqrtD = 0.08838834764831845f;  // 1 / sqrt(128), correctly rounded

typedef uint16_t bf16_t;  // bfloat16 kept as its raw bit pattern

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bfloat16, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

// Eight consecutive elements of a row in their storage format.  A lane owns
// one such slice; 16 lanes cover a 128-wide row.
template <typename T>
struct Slice8;

template <>
struct Slice8<bf16_t> {
    uint4 raw;
    __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
    __device__ __forceinline__ void zero() { raw = make_uint4(0, 0, 0, 0); }
    __device__ __forceinline__ void unpack(float* x) const {
        x[0] = bf16_lo(raw.x); x[1] = bf16_hi(raw.x);
        x[2] = bf16_lo(raw.y); x[3] = bf16_hi(raw.y);
        x[4] = bf16_lo(raw.z); x[5] = bf16_hi(raw.z);
        x[6] = bf16_lo(raw.w); x[7] = bf16_hi(raw.w);
    }
    __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = raw; }
};

template <>
struct Slice8<float> {
    float4 a, b;
    __device__ __forceinline__ void load(const float* p) {
        a = *reinterpret_cast<const float4*>(p);
        b = *reinterpret_cast<const float4*>(p + 4);
    }
    __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
    __device__ __forceinline__ void unpack(float* x) const {
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
    }
    __device__ __forceinline__ void store(float* p) const {
        *reinterpret_cast<float4*>(p) = a;
        *reinterpret_cast<float4*>(p + 4) = b;
    }
};

// Stores 8 floats rounded to the storage format.
__device__ __forceinline__ void store8(bf16_t* p, const float* x) {
    uint4 r;
    r.x = f32_to_bf16_bits(x[0]) | (f32_to_bf16_bits(x[1]) << 16);
    r.y = f32_to_bf16_bits(x[2]) | (f32_to_bf16_bits(x[3]) << 16);
    r.z = f32_to_bf16_bits(x[4]) | (f32_to_bf16_bits(x[5]) << 16);
    r.w = f32_to_bf16_bits(x[6]) | (f32_to_bf16_bits(x[7]) << 16);
    *reinterpret_cast<uint4*>(p) = r;
}
__device__ __forceinline__ void store8(float* p, const float* x) {
    *reinterpret_cast<float4*>(p) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}

// Sum over each row of 16 lanes with DPP moves; every lane of the row ends
// with the same bits (each step adds two equal-valued partners commutatively).
#define MPA_DPP(v, ctrl) \
    __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), (ctrl), 0xF, 0xF, true))
__device__ __forceinline__ float row16_sum(float v) {
    v += MPA_DPP(v, 0xB1);   // quad_perm [1,0,3,2]
    v += MPA_DPP(v, 0x4E);   // quad_perm [2,3,0,1]
    v += MPA_DPP(v, 0x141);  // row_half_mirror
    v += MPA_DPP(v, 0x140);  // row_mirror
    return v;
}

__device__ __forceinline__ float shfl_xor_f(float v, int mask) { return __shfl_xor(v, mask, kWave); }
__device__ __forceinline__ int shfl_xor_i(int v, int mask) { return __shfl_xor(v, mask, kWave); }

// Workgroups are dispatched round-robin over the XCDs.  This maps hardware
// workgroup id `bid` (grid padded to a multiple of kXcds) to a logical id such
// that consecutive logical ids run on the same XCD and share its L2.
__device__ __forceinline__ int xcd_logical_id(int bid, int grid) {
    const int per_xcd = grid / kXcds;
    return (bid % kXcds) * per_xcd + bid / kXcds;
}

// splitmix64 finaliser (Steele, Lea & Flood 2014).
__device__ __forceinline__ uint64_t sm64_mix(uint64_t z) {
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
constexpr uint64_t kSm64Gamma = 0x9E3779B97F4A7C15ull;

// Inclusive sum over the 64 lanes of a wave with DPP moves: shifts by 1, 2,
// 4 and 8 lanes inside each row of 16, then the last lane of row 0 (and 2) is
// broadcast into rows 1 and 3, and the last lane of row 1 into rows 2 and 3.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15 -> rows 1, 3
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31 -> rows 2, 3
    return v;
}

// Value of lane `src` (uniform) in every lane.
__device__ __forceinline__ int lane_value(int v, int src) { return __builtin_amdgcn_readlane(v, src); }

// Exclusive prefix sums of four ints over a 256-thread workgroup, in thread
// order; `totals` receives the four sums.  Uses 4 * 4 ints of LDS.
__device__ __forceinline__ int4 block256_exclusive_sum4(int4 v, int4& totals, int* lds16) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = threadIdx.x / kWave;
    int4 inc;
    inc.x = wave_inclusive_sum(v.x);
    inc.y = wave_inclusive_sum(v.y);
    inc.z = wave_inclusive_sum(v.z);
    inc.w = wave_inclusive_sum(v.w);
    if (lane == kWave - 1) {
        lds16[wave * 4 + 0] = inc.x;
        lds16[wave * 4 + 1] = inc.y;
        lds16[wave * 4 + 2] = inc.z;
        lds16[wave * 4 + 3] = inc.w;
    }
    __syncthreads();
    int4 base = make_int4(0, 0, 0, 0);
    totals = make_int4(0, 0, 0, 0);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        int4 t = make_int4(lds16[w * 4 + 0], lds16[w * 4 + 1], lds16[w * 4 + 2], lds16[w * 4 + 3]);
        if (w < wave) {
            base.x += t.x; base.y += t.y; base.z += t.z; base.w += t.w;
        }
        totals.x += t.x; totals.y += t.y; totals.z += t.z; totals.w += t.w;
    }
    __syncthreads();  // lds16 may be reused right after
    return make_int4(base.x + inc.x - v.x, base.y + inc.y - v.y, base.z + inc.z - v.z, base.w + inc.w - v.w);
}

// The query slice of one head: bf16 pairs for the packed dot product, or fp32.
template <typename T>
struct QSlice;
template <>
struct QSlice<bf16_t> {
    uint4 raw;
    __device__ __forceinline__ void load(const bf16_t* p) { raw = *reinterpret_cast<const uint4*>(p); }
};
template <>
struct QSlice<float> {
    float v[8];
    __device__ __forceinline__ void load(const float* p) {
        Slice8<float> s;
        s.load(p);
        s.unpack(v);
    }
};

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Partial dot product of a lane's 8 elements (fp32 accumulation).
__device__ __forceinline__ float dot8(const QSlice<bf16_t>& q, const Slice8<bf16_t>& k) {
    float d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.raw.x),
                                              __builtin_bit_cast(bf16x2_t, k.raw.x), 0.f, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.raw.y), __builtin_bit_cast(bf16x2_t, k.raw.y),
                                        d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.raw.z), __builtin_bit_cast(bf16x2_t, k.raw.z),
                                        d, false);
    d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, q.raw.w), __builtin_bit_cast(bf16x2_t, k.raw.w),
                                        d, false);
    return d;
}
__device__ __forceinline__ float dot8(const QSlice<float>& q, const Slice8<float>& k) {
    float x[8];
    k.unpack(x);
    float d = q.v[0] * x[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) d = fmaf(q.v[e], x[e], d);
    return d;
}

}  // namespace mpa
