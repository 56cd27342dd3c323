// codes.hip -- fp8 copies of the centroid rows for the decode: E4M3 codes
// (OCP 8-bit floating point: bias 7, 3 mantissa bits, subnormals, largest
// finite 448) with one power-of-two scale per 32 values, stored as the byte
// E + 127.  E is the least integer >= -126 with max|x| * 2^-E <= 448, so no
// value is clamped; each code is the E4M3 value nearest to x * 2^-E, ties to
// the even code, with the sign bit of x.
//
// The pages keep the centroids in the cache's precision; these copies halve
// the centroid bytes a decode step reads (the k-means keeps using the stored
// centroids).
#include <math.h>

#include "device.hpp"
#include "kernels.hpp"

namespace mpa {

// Scale exponent of a block from its largest magnitude (exact: exponent and
// mantissa bits of the float).
__device__ __forceinline__ int block_exponent(float amax) {
    const uint32_t u = __float_as_uint(amax);
    const int ef = (int)(u >> 23);
    if (ef == 0) return -126;                       // zero or below 2^-126: the floor
    int E = ef - 127 - 8;                           // amax * 2^-E in [256, 512)
    if ((u & 0x7FFFFFu) > 0x600000u) ++E;           // above 1.75 * 2^8 = 448
    return E < -126 ? -126 : E;
}

// E4M3 code of y = x * 2^-E (|y| <= 448, exact in fp32 or below 2^-126).
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const uint32_t sign = (__float_as_uint(y) >> 24) & 0x80u;
    const float a = fabsf(y);
    uint32_t mag;
    if (a < 0x1p-6f) {
        mag = (uint32_t)rintf(a * 512.f);          // subnormal steps of 2^-9 (8: the least normal)
    } else {
        const uint32_t ua = __float_as_uint(a);
        const uint32_t r = ua + 0x7FFFFu + ((ua >> 20) & 1u);  // 3 mantissa bits, ties to even
        mag = (((r >> 23) - 120u) << 3) | ((r >> 20) & 7u);    // exponent bias 127 -> 7
    }
    return sign | mag;
}

// One thread per 32-value block: row c_begin + t / 8 of each unit, blocks
// 0-3 of the key row, then 0-3 of the value row.
__global__ __launch_bounds__(256) void encode_codes_kernel(UnitGeom g, int c_begin, int c_count,
                                                           const bf16_t* __restrict__ kbar,
                                                           const bf16_t* __restrict__ vbar,
                                                           uint8_t* __restrict__ kcodes, uint8_t* __restrict__ kscales,
                                                           uint8_t* __restrict__ vcodes, uint8_t* __restrict__ vscales) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    const int unit = blockIdx.y;
    const int c = c_begin + (t >> 3), part = t & 7;
    if (c >= c_begin + c_count) return;
    const bool key = part < 4;
    const int blk = part & 3;
    const size_t row = (size_t)unit * g.Cmax + c;
    const bf16_t* src = (key ? kbar : vbar) + row * kHeadDim + blk * 32;
    float x[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        Slice8<bf16_t> s;
        s.load(src + q * 8);
        s.unpack(x + q * 8);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    const int E = block_exponent(amax);
    const float inv = __uint_as_float((uint32_t)(127 - E) << 23);  // 2^-E, E in [-126, 121]
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        uint32_t v = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) v |= e4m3_code(x[q * 4 + e] * inv) << (8 * e);
        w[q] = v;
    }
    uint8_t* dst = (key ? kcodes : vcodes) + row * kHeadDim + blk * 32;
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    (key ? kscales : vscales)[row * (kHeadDim / 32) + blk] = (uint8_t)(E + 127);
}

hipError_t launch_encode_codes(UnitGeom g, int c_begin, int c_count, const void* kbar, const void* vbar,
                               uint8_t* kcodes, uint8_t* kscales, uint8_t* vcodes, uint8_t* vscales, hipStream_t st) {
    if (c_count <= 0) return hipSuccess;
    dim3 grid((unsigned)(((int64_t)c_count * 8 + 255) / 256), g.units);
    hipLaunchKernelGGL(encode_codes_kernel, grid, dim3(256), 0, st, g, c_begin, c_count, (const bf16_t*)kbar,
                       (const bf16_t*)vbar, kcodes, kscales, vcodes, vscales);
    return hipGetLastError();
}

}  // namespace mpa
