// lmhead_kernels.h — greedy verification straight from the target's hidden
// states: the unembedding product ("FlashMap: Flow Map Speculative Decoding
// and the Mathematical Elimination of Suffix Decay", section 3: the logits of
// a position are its hidden state times the transposed unembedding matrix)
// is computed tile by tile with matrix-core instructions (bf16 inputs, fp32
// accumulation) and every tile is reduced in registers to its per-row
// maximum and the lowest token index holding it, so no logit is written to
// memory.  The greedy rule of "DFlash", section 4, then runs on the argmax.
//
//  k_lmhead_argmax : one 256-thread workgroup per (128 rows, 256 tokens)
//                    tile; 64-wide steps along the hidden dimension staged
//                    through LDS, the next step's operands loaded into
//                    registers while the current one multiplies; each wave
//                    owns a 64 x 128 block (2 x 4 v_mfma_f32_32x32x16_bf16);
//                    writes one (max, index) pair per (row, vocabulary tile).
//  k_lmhead_merge  : one workgroup per row: the argmax over its tile pairs.
//
// MFMA 32x32x16 operand layout (lane l, element j of the 8-element operand,
// measured): A[m = l % 32][k = 8 (l / 32) + j], B[k = 8 (l / 32) + j][n = l % 32];
// result element i holds D[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32].
#pragma once

#include <cstdint>

#include "device_common.h"

namespace sv {

constexpr int kLmM = 128;   // rows per workgroup tile
constexpr int kLmN = 256;   // tokens per workgroup tile
constexpr int kLmNI = kLmN / 64;  // 32-token MFMA blocks per wave (two waves across the tokens)
constexpr int kLmK = 64;    // hidden elements per step
constexpr int kLmPad = 8;   // LDS row padding (bf16 elements)

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_float16 __attribute__((ext_vector_type(16)));

struct LmPart {
    float v;  // tile maximum of the row
    int i;    // lowest token index holding it (INT32_MAX: none)
};

struct LmArgs {
    const uint16_t* hidden;  // [R][H] bf16
    const uint16_t* w;       // [V][H] bf16
    int R, V, H;
    int n_vt;                // vocabulary tiles, ceil(V / kLmN)
    int n_rt;                // row tiles, ceil(R / kLmM)
    LmPart* part;            // [R][n_vt]
    int32_t* gidx;           // [R]
};

// (v, i) better than (bv, bi): larger value, or equal value at a lower index.
__device__ __forceinline__ bool lm_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

__global__ void __launch_bounds__(256, 2) k_lmhead_argmax(LmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[kLmM][kLmK + kLmPad];
    __shared__ __attribute__((aligned(16))) uint16_t sW[kLmN][kLmK + kLmPad];
    __shared__ LmPart sP[kLmM][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    // Workgroups are dispatched to the 8 XCDs in turn (workgroup L to XCD
    // L mod 8), each XCD with its own L2.  Workgroup L = 8 (n_rt q + rt) + x
    // takes row tile rt of vocabulary tile 8 q + x, so every row tile of a
    // vocabulary tile runs on one XCD at about the same time and the
    // unembedding rows come from HBM once.
    const int L = blockIdx.x, x = L & 7, qr = L >> 3;
    const int rt = qr % a.n_rt, vt = (qr / a.n_rt) * 8 + x;
    if (vt >= a.n_vt) return;
    const int row0 = rt * kLmM, v0 = vt * kLmN;
    lm_float16 acc[2][kLmNI];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < kLmNI; ++ni)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;

    // one step stages 128 x kLmK of each operand: pieces of 8 bf16, kLmK / 8
    // per row, kPieces per thread; rows past R or V and columns past H read
    // as zero (no memory access)
    constexpr int kPerRow = kLmK / 8;
    constexpr int kPiecesA = kLmM * kPerRow / 256;
    constexpr int kPiecesW = kLmN * kPerRow / 256;
    uint4 ra[kPiecesA], rw[kPiecesW];
    auto load = [&](int h0) {
#pragma unroll
        for (int q = 0; q < kPiecesA; ++q) {
            const int e = tid + q * 256;
            const int r = e / kPerRow, hh = h0 + (e % kPerRow) * 8;
            ra[q] = make_uint4(0u, 0u, 0u, 0u);
            if (row0 + r < a.R && hh < a.H) ra[q] = *reinterpret_cast<const uint4*>(a.hidden + (size_t)(row0 + r) * a.H + hh);
        }
#pragma unroll
        for (int q = 0; q < kPiecesW; ++q) {
            const int e = tid + q * 256;
            const int r = e / kPerRow, hh = h0 + (e % kPerRow) * 8;
            rw[q] = make_uint4(0u, 0u, 0u, 0u);
            if (v0 + r < a.V && hh < a.H) rw[q] = *reinterpret_cast<const uint4*>(a.w + (size_t)(v0 + r) * a.H + hh);
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int q = 0; q < kPiecesA; ++q) {
            const int e = tid + q * 256;
            *reinterpret_cast<uint4*>(&sA[e / kPerRow][(e % kPerRow) * 8]) = ra[q];
        }
#pragma unroll
        for (int q = 0; q < kPiecesW; ++q) {
            const int e = tid + q * 256;
            *reinterpret_cast<uint4*>(&sW[e / kPerRow][(e % kPerRow) * 8]) = rw[q];
        }
    };
    load(0);
    for (int h0 = 0; h0 < a.H; h0 += kLmK) {
        store();
        __syncthreads();
        load(h0 + kLmK);  // the next step's operands arrive while this one multiplies
#pragma unroll
        for (int ks = 0; ks < kLmK / 16; ++ks) {
            const int kc = ks * 16 + (lane >> 5) * 8;
            lm_bf16x8 fa[2], fb[kLmNI];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                fa[mi] = __builtin_bit_cast(lm_bf16x8, *reinterpret_cast<const uint4*>(&sA[wm * 64 + mi * 32 + (lane & 31)][kc]));
#pragma unroll
            for (int ni = 0; ni < kLmNI; ++ni)
                fb[ni] = __builtin_bit_cast(lm_bf16x8, *reinterpret_cast<const uint4*>(&sW[wn * (kLmN / 2) + ni * 32 + (lane & 31)][kc]));
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < kLmNI; ++ni)
                    acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
        }
        __syncthreads();
    }

    // per row of this wave's block: the best over its 64 tokens (the two
    // column blocks, then the 32 lanes of the half-wave holding the row)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int n0 = v0 + wn * (kLmN / 2) + (lane & 31);
            float bv = n0 < a.V ? acc[mi][0][i] : -INFINITY;
            int bi = n0 < a.V ? n0 : INT32_MAX;
#pragma unroll
            for (int ni = 1; ni < kLmNI; ++ni) {
                const int n1 = n0 + 32 * ni;
                if (n1 < a.V && lm_better(acc[mi][ni][i], n1, bv, bi)) {
                    bv = acc[mi][ni][i];
                    bi = n1;
                }
            }
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oi = __shfl_xor(bi, off);
                if (lm_better(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((lane & 31) == 0) sP[wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][wn] = LmPart{bv, bi};
        }
    }
    __syncthreads();
    if (tid < kLmM && row0 + tid < a.R) {
        LmPart p = sP[tid][0];
        const LmPart q = sP[tid][1];
        if (lm_better(q.v, q.i, p.v, p.i)) p = q;
        a.part[(size_t)(row0 + tid) * a.n_vt + vt] = p;
    }
}

__global__ void __launch_bounds__(256) k_lmhead_merge(LmArgs a) {
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const LmPart* p = a.part + (size_t)row * a.n_vt;
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int t = tid; t < a.n_vt; t += 256) {
        const LmPart q = p[t];
        if (lm_better(q.v, q.i, bv, bi)) {
            bv = q.v;
            bi = q.i;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off);
        const int oi = __shfl_xor(bi, off);
        if (lm_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        s_v[wave] = bv;
        s_i[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w2 = 1; w2 < 4; ++w2)
            if (lm_better(s_v[w2], s_i[w2], bv, bi)) {
                bv = s_v[w2];
                bi = s_i[w2];
            }
        a.gidx[row] = bi;
    }
}

}  // namespace sv
