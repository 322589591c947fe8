// lmhead_kernels.h — the unembedding product on the matrix cores: a
// position's logits are its hidden state times the transposed unembedding
// matrix ("FlashMap: Flow Map Speculative Decoding and the Mathematical
// Elimination of Suffix Decay", section 3; the drafter reuses the target's
// LM head, FlashMap section 5 and "DFlash" section 5), computed tile by tile
// with bf16 products accumulated in fp32.  Two epilogues:
//
//  argmax : each tile is reduced in registers to its per-row maximum and the
//           lowest token index holding it, so no logit is written to memory
//           (greedy verification, the greedy rule of "DFlash" section 4);
//           k_lmhead_merge then takes each row's argmax over its tiles.
//  store  : the tile's logits are rounded to bf16 (nearest, ties to even, as
//           a bf16 LM head outputs them) and stored, for the sampling path.
//
// k_lmhead<EPI> is persistent: exactly the workgroups the GPU holds at once,
// each looping over (128 rows, 256 tokens) tiles in an XCD-aware order.  A
// tile walks the hidden dimension in 32-wide steps through two LDS buffers:
// the operands of the next two steps are loaded into registers while the
// current step multiplies, and the next step's are stored into the other
// buffer afterwards, so each step needs one barrier.  Each of the 4 waves owns a 64 x 128 block
// (2 x 4 v_mfma_f32_32x32x16_bf16 per 16-wide slice).
//
// MFMA 32x32x16 operand layout (lane l, element j of the 8-element operand,
// measured): A[m = l % 32][k = 8 (l / 32) + j], B[k = 8 (l / 32) + j][n = l % 32];
// result element i holds D[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32].
#pragma once

#include <cstdint>

#include "device_common.h"

namespace sv {

constexpr int kLmM = 128;   // rows per tile
constexpr int kLmN = 256;   // tokens per tile
constexpr int kLmNI = kLmN / 64;  // 32-token MFMA blocks per wave (two waves across the tokens)
constexpr int kLmK = 32;    // hidden elements per step
constexpr int kLmPad = 8;   // LDS row padding (bf16 elements)
constexpr int kLmThreads = 256;
constexpr int kLmPerCU = 2; // workgroups a compute unit holds (LDS)

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_float16 __attribute__((ext_vector_type(16)));

struct LmPart {
    float v;  // tile maximum of the row
    int i;    // lowest token index holding it (INT32_MAX: none)
};

struct LmArgs {
    const uint16_t* hidden;   // rows [0, R1): [R1][H] bf16
    const uint16_t* hidden2;  // rows [R1, R): [R - R1][H] bf16 (unused when R1 == R)
    int R1;
    const uint16_t* w;        // [V][H] bf16
    int R, V, H;
    int n_vt;                 // vocabulary tiles, ceil(V / kLmN)
    int n_rt;                 // row tiles, ceil(R / kLmM)
    int n_tiles;              // tile slots: ceil(n_vt / 8) * 8 * n_rt
    LmPart* part;             // argmax: [R][n_vt]
    int32_t* gidx;            // argmax: [R]
    uint16_t* logits;         // store: [R][V] bf16
};

enum { LM_ARGMAX = 0, LM_STORE = 1 };

// (v, i) better than (bv, bi): larger value, or equal value at a lower index.
__device__ __forceinline__ bool lm_better(float v, int i, float bv, int bi) { return v > bv || (v == bv && i < bi); }

// bf16 bits of a finite float, rounded to nearest, ties to even.
__device__ __forceinline__ uint16_t lm_bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <int EPI>
__global__ void __launch_bounds__(kLmThreads, kLmPerCU) k_lmhead(LmArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kLmM][kLmK + kLmPad];
    __shared__ __attribute__((aligned(16))) uint16_t sW[2][kLmN][kLmK + kLmPad];
    __shared__ LmPart sP[kLmM][2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    constexpr int kPerRow = kLmK / 8;                        // 16-byte pieces per row and step
    constexpr int kPiecesA = kLmM * kPerRow / kLmThreads;    // 2
    constexpr int kPiecesW = kLmN * kPerRow / kLmThreads;    // 4
    const int n_steps = (a.H + kLmK - 1) / kLmK;
    // Tile slot T = 8 (n_rt q + rt) + x holds row tile rt of vocabulary tile
    // 8 q + x.  Workgroups are dispatched to the 8 XCDs in turn (workgroup L
    // to XCD L mod 8, each XCD with its own L2) and the grid is a multiple of
    // 8, so slot T always runs on XCD T mod 8: every row tile of a vocabulary
    // tile runs on one XCD at about the same time and the unembedding rows
    // come from HBM once.
    for (int T = blockIdx.x; T < a.n_tiles; T += gridDim.x) {
        const int x = T & 7, qr = T >> 3;
        const int rt = qr % a.n_rt, vt = (qr / a.n_rt) * 8 + x;
        if (vt >= a.n_vt) continue;  // padding slot (uniform over the workgroup)
        const int row0 = rt * kLmM, v0 = vt * kLmN;
        lm_float16 acc[2][kLmNI];
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
            for (int ni = 0; ni < kLmNI; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
        // rows past R or V and columns past H read as zero (no memory access)
        struct Stage {
            uint4 a[kPiecesA], w[kPiecesW];
        };
        auto load = [&](int h0, Stage& g) {
#pragma unroll
            for (int q = 0; q < kPiecesA; ++q) {
                const int e = tid + q * kLmThreads;
                const int r = row0 + e / kPerRow, hh = h0 + (e % kPerRow) * 8;
                g.a[q] = make_uint4(0u, 0u, 0u, 0u);
                if (r < a.R && hh < a.H) {
                    const uint16_t* hp = r < a.R1 ? a.hidden + (size_t)r * a.H : a.hidden2 + (size_t)(r - a.R1) * a.H;
                    g.a[q] = *reinterpret_cast<const uint4*>(hp + hh);
                }
            }
#pragma unroll
            for (int q = 0; q < kPiecesW; ++q) {
                const int e = tid + q * kLmThreads;
                const int r = v0 + e / kPerRow, hh = h0 + (e % kPerRow) * 8;
                g.w[q] = make_uint4(0u, 0u, 0u, 0u);
                if (r < a.V && hh < a.H) g.w[q] = *reinterpret_cast<const uint4*>(a.w + (size_t)r * a.H + hh);
            }
        };
        auto store = [&](int buf, const Stage& g) {
#pragma unroll
            for (int q = 0; q < kPiecesA; ++q) {
                const int e = tid + q * kLmThreads;
                *reinterpret_cast<uint4*>(&sA[buf][e / kPerRow][(e % kPerRow) * 8]) = g.a[q];
            }
#pragma unroll
            for (int q = 0; q < kPiecesW; ++q) {
                const int e = tid + q * kLmThreads;
                *reinterpret_cast<uint4*>(&sW[buf][e / kPerRow][(e % kPerRow) * 8]) = g.w[q];
            }
        };
        auto compute = [&](int cur) {
#pragma unroll
            for (int ks = 0; ks < kLmK / 16; ++ks) {
                const int kc = ks * 16 + (lane >> 5) * 8;
                lm_bf16x8 fa[2], fb[kLmNI];
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
                    fa[mi] = __builtin_bit_cast(
                        lm_bf16x8, *reinterpret_cast<const uint4*>(&sA[cur][wm * 64 + mi * 32 + (lane & 31)][kc]));
#pragma unroll
                for (int ni = 0; ni < kLmNI; ++ni)
                    fb[ni] = __builtin_bit_cast(
                        lm_bf16x8,
                        *reinterpret_cast<const uint4*>(&sW[cur][wn * (kLmN / 2) + ni * 32 + (lane & 31)][kc]));
#pragma unroll
                for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                    for (int ni = 0; ni < kLmNI; ++ni)
                        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
            }
        };
        // Loads run two steps ahead in two register stages: step s multiplies
        // buffer s & 1 while the loads of steps s + 1 (issued during step s - 1)
        // and s + 2 (issued now) are in flight; the stage of step s + 1 is
        // stored into the other buffer, last read in step s - 1, after the
        // multiply.  Steps are unrolled in pairs so that the register stages
        // stay fixed.
        Stage g0, g1;
        load(0, g0);
        if (n_steps > 1) load(kLmK, g1);
        store(0, g0);
        __syncthreads();
        for (int s = 0; s < n_steps; s += 2) {
            // step s: buffer 0; g1 holds step s + 1
            if (s + 2 < n_steps) load((s + 2) * kLmK, g0);
            compute(0);
            if (s + 1 < n_steps) store(1, g1);
            __syncthreads();
            if (s + 1 >= n_steps) break;
            // step s + 1: buffer 1; g0 holds step s + 2
            if (s + 3 < n_steps) load((s + 3) * kLmK, g1);
            compute(1);
            if (s + 2 < n_steps) store(0, g0);
            __syncthreads();
        }

        if constexpr (EPI == LM_STORE) {
            // bf16 logits: lanes of a half-wave hold 32 consecutive tokens of one row
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int ni = 0; ni < kLmNI; ++ni)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = row0 + wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                        const int n = v0 + wn * (kLmN / 2) + ni * 32 + (lane & 31);
                        if (r < a.R && n < a.V) a.logits[(size_t)r * a.V + n] = lm_bf16_rne(acc[mi][ni][i]);
                    }
        } else {
            // per row of this wave's block: the best over its 128 tokens (the
            // four column blocks, then the 32 lanes of the half-wave holding the row)
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
                    if ((lane & 31) == 0)
                        sP[wm * 64 + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][wn] = LmPart{bv, bi};
                }
            }
            __syncthreads();
            if (tid < kLmM && row0 + tid < a.R) {
                LmPart p = sP[tid][0];
                const LmPart q = sP[tid][1];
                if (lm_better(q.v, q.i, p.v, p.i)) p = q;
                a.part[(size_t)(row0 + tid) * a.n_vt + vt] = p;
            }
            __syncthreads();  // sP is written again by the next tile
        }
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
