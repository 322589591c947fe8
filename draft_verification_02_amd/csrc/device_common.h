// device_common.h — small device helpers shared by the verification kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kBlock = 256;       // threads per workgroup (4 wave64)
constexpr int kWaves = kBlock / 64;
constexpr int kEPT = 32;          // elements per thread per streaming tile
constexpr int kTile = kBlock * kEPT;  // 8192 elements per streaming tile

enum { DT_F32 = 0, DT_BF16 = 1 };

// Arrival counters that many workgroups add to sit one per 256 bytes: atomics
// on one cache line serialize even when their addresses differ (measured: 32
// per-sequence counters packed in one line took the 4768-workgroup draw of a
// 32-tree batch from about 18 to 63 us).
constexpr int kCntStride = 64;  // unsigned ints

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load marked non-temporal (data is read once).
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// One stored logit, widened to float (exact for both formats).
__device__ __forceinline__ float load_logit(const char* row, int dt, long long i) {
    if (dt == DT_F32) return reinterpret_cast<const float*>(row)[i];
    const uint32_t h = reinterpret_cast<const uint16_t*>(row)[i];
    return __uint_as_float(h << 16);
}

// Order-preserving 32-bit key of a float: a < b  <=>  key(a) < key(b) for
// non-NaN values; -0 and +0 map to the same key.
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f);
    u = (u == 0x80000000u) ? 0u : u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
    const uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
    return __uint_as_float(u);
}

// ---- cross-lane moves within a wave64, by DPP (no LDS round trip) --------
// Every helper below expects all 64 lanes active.
enum : int {
    kDppQuadXor1 = 0xB1,       // quad_perm [1,0,3,2]: lane ^ 1
    kDppQuadXor2 = 0x4E,       // quad_perm [2,3,0,1]: lane ^ 2
    kDppRowMirror = 0x140,     // lane 15 - i within a row of 16
    kDppRowHalfMirror = 0x141, // lane 7 - i within a half row of 8
    kDppRowShr1 = 0x111,
    kDppRowShr2 = 0x112,
    kDppRowShr4 = 0x114,
    kDppRowShr8 = 0x118,
    kDppRowBcast15 = 0x142,    // lane 15 of each row to the next row
    kDppRowBcast31 = 0x143,    // lane 31 to rows 2 and 3
    kDppWaveShr1 = 0x138,      // lane i - 1 of the whole wave
};

template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    // lanes outside ROWS, or whose source lies outside the row, read 0
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xF, ZERO);
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ unsigned long long dpp_u64(unsigned long long v) {
    const uint32_t lo = dpp_u32<CTRL, ROWS, ZERO>((uint32_t)v);
    const uint32_t hi = dpp_u32<CTRL, ROWS, ZERO>((uint32_t)(v >> 32));
    return ((unsigned long long)hi << 32) | lo;
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ float dpp_move(float v) {
    return __uint_as_float(dpp_u32<CTRL, ROWS, ZERO>(__float_as_uint(v)));
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ int dpp_move(int v) {
    return (int)dpp_u32<CTRL, ROWS, ZERO>((uint32_t)v);
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ uint32_t dpp_move(uint32_t v) {
    return dpp_u32<CTRL, ROWS, ZERO>(v);
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ unsigned long long dpp_move(unsigned long long v) {
    return dpp_u64<CTRL, ROWS, ZERO>(v);
}
template <int CTRL, int ROWS = 0xF, bool ZERO = true>
__device__ __forceinline__ double dpp_move(double v) {
    return __longlong_as_double((long long)dpp_u64<CTRL, ROWS, ZERO>((unsigned long long)__double_as_longlong(v)));
}

// The value of `lane` (a wave-uniform lane number) in every lane.
__device__ __forceinline__ uint32_t lane_read(uint32_t v, int lane) {
    return (uint32_t)__builtin_amdgcn_readlane((int)v, lane);
}
__device__ __forceinline__ int lane_read(int v, int lane) { return __builtin_amdgcn_readlane(v, lane); }
__device__ __forceinline__ float lane_read(float v, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
__device__ __forceinline__ unsigned long long lane_read(unsigned long long v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((unsigned long long)hi << 32) | lo;
}
__device__ __forceinline__ double lane_read(double v, int lane) {
    return __longlong_as_double((long long)lane_read((unsigned long long)__double_as_longlong(v), lane));
}

// op over the wave, the same value in every lane: butterflies inside each
// row of 16 (commutative steps, so every lane of a row ends equal), then the
// four row values combined in a fixed order.
template <class T, class Op>
__device__ __forceinline__ T wave_allreduce(T v, Op op) {
    v = op(v, dpp_move<kDppQuadXor1>(v));
    v = op(v, dpp_move<kDppQuadXor2>(v));
    v = op(v, dpp_move<kDppRowHalfMirror>(v));
    v = op(v, dpp_move<kDppRowMirror>(v));
    return op(op(lane_read(v, 0), lane_read(v, 16)), op(lane_read(v, 32), lane_read(v, 48)));
}

// Inclusive prefix sum in lane order (within rows by doubling, then across
// rows by broadcasts); a fixed order of additions.
template <class T>
__device__ __forceinline__ T wave_incl_scan(T x) {
    x = x + dpp_move<kDppRowShr1>(x);
    x = x + dpp_move<kDppRowShr2>(x);
    x = x + dpp_move<kDppRowShr4>(x);
    x = x + dpp_move<kDppRowShr8>(x);
    x = x + dpp_move<kDppRowBcast15, 0xA>(x);
    x = x + dpp_move<kDppRowBcast31, 0xC>(x);
    return x;
}
// The previous lane's value (0 in lane 0).
template <class T>
__device__ __forceinline__ T wave_shift_up1(T x) {
    return dpp_move<kDppWaveShr1>(x);
}

// ---- wave64 reductions (fixed combination order, hence deterministic) ----
__device__ __forceinline__ float wave_max(float v) {
    return wave_allreduce(v, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ double wave_sum(double v) {
    return wave_allreduce(v, [](double a, double b) { return a + b; });
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
    return wave_allreduce(v, [](unsigned long long a, unsigned long long b) { return a > b ? a : b; });
}

// Block-wide max / sum over kBlock threads through LDS (fixed order).
__device__ __forceinline__ float block_max(float v, float* s4) {
    v = wave_max(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s4[wid] = v;
    __syncthreads();
    float r = s4[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r = fmaxf(r, s4[w]);
    return r;
}
__device__ __forceinline__ double block_sum(double v, double* s4) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s4[wid] = v;
    __syncthreads();
    double r = s4[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) r += s4[w];
    return r;
}

// ---- Philox4x32-10 -------------------------------------------------------
// Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3"
// (SC'11): ten rounds; each multiplies counter words 0 and 2 by the round
// constants, splits the products into high and low halves and mixes the high
// halves with words 1 and 3 and the key; the key advances by the Weyl
// constants between rounds.
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox4x32_10(U4 c, uint32_t k0, uint32_t k1) {
    constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t hi0 = __umulhi(M0, c.x), lo0 = M0 * c.x;
        const uint32_t hi1 = __umulhi(M1, c.z), lo1 = M1 * c.z;
        c = U4{hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0};
        k0 += W0;
        k1 += W1;
    }
    return c;
}

enum { PURPOSE_ACCEPT = 0, PURPOSE_SAMPLE = 1 };

__device__ __forceinline__ U4 draw_block(uint64_t seed, uint32_t b, uint32_t k, uint32_t purpose) {
    return philox4x32_10(U4{b, k, purpose, 0u}, static_cast<uint32_t>(seed),
                         static_cast<uint32_t>(seed >> 32));
}
// 24-bit uniform in [0, 1) from word 0.
__device__ __forceinline__ double uniform24(U4 w) { return (double)(w.x >> 8) * 0x1p-24; }
// 53-bit uniform in [0, 1) from words 0 and 1 (27 + 26 bits).
__device__ __forceinline__ double uniform53(U4 w) {
    return ((double)(w.x >> 5) * 67108864.0 + (double)(w.y >> 6)) * 0x1p-53;
}

}  // namespace sv
