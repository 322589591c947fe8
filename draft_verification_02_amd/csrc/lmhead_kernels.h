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
// k_lmhead<EPI> is persistent: one workgroup of 8 waves per compute unit,
// each looping over (256 rows, 320 tokens) tiles (see the schedule below).
// A tile spans 256 rows so that, for up to 256 rows (a batch of 32 sequences
// of 8 positions), every unembedding row is read from memory by one
// workgroup only.  Every tile re-reads the hidden states (from L2), and 320
// tokens, the widest tile whose accumulators fit the registers of 8 waves,
// spread that re-read over the most tokens.  A tile
// walks the hidden dimension in 32-wide steps through a ring of four LDS
// stages that the loads fill directly (global_load_lds_dwordx4: no registers
// hold loaded data), so three steps are in flight while the fourth
// multiplies and each step needs one barrier.  Each wave owns 64 rows x 160
// tokens (2 x 5 v_mfma_f32_32x32x16_bf16 per 16-wide slice).
//
// MFMA 32x32x16 operand layout (lane l, element j of the 8-element operand,
// measured): A[m = l % 32][k = 8 (l / 32) + j], B[k = 8 (l / 32) + j][n = l % 32];
// result element i holds D[m = 8 (i / 4) + 4 (l / 32) + i % 4][n = l % 32].
// A direct-to-LDS load writes lane l's 16 bytes at the wave's LDS base plus
// 16 l (measured).
#pragma once

#include <cstdint>
#include <type_traits>

#include "device_common.h"
#include "seq_kernels.h"

namespace sv {

constexpr int kLmM = 256;   // rows per tile
constexpr int kLmN = 320;   // tokens per tile
constexpr int kLmWM = 4;    // waves across the rows
constexpr int kLmWN = 2;    // waves across the tokens
constexpr int kLmMI = kLmM / kLmWM / 32;  // 32-row MFMA blocks per wave
constexpr int kLmNI = kLmN / kLmWN / 32;  // 32-token MFMA blocks per wave
constexpr int kLmK = 32;    // hidden elements per step
constexpr int kLmThreads = 64 * kLmWM * kLmWN;
constexpr int kLmWaves = kLmThreads / 64;
constexpr int kLmPerCU = 1; // workgroups a compute unit holds (LDS)
constexpr int kLmStages = 4;                      // LDS ring depth
constexpr int kLmChunks = kLmK / 8;               // 16-byte chunks per row and step
constexpr int kLmStageA = kLmM * kLmChunks;       // chunks of hidden state per stage
constexpr int kLmStage = (kLmM + kLmN) * kLmChunks;  // chunks per stage (36 KiB)
constexpr int kLmBlkW = kLmN * kLmChunks / 64;    // 64-chunk load blocks of unembedding rows per step
static_assert(kLmM * kLmChunks % (kLmThreads * 2) == 0, "a half tile's hidden rows split evenly over the waves");
static_assert(kLmN * kLmChunks % 64 == 0, "whole load blocks");

typedef __bf16 lm_bf16x8 __attribute__((ext_vector_type(8)));
typedef float lm_float16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lm_lds_void;

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
    LmPart* part;             // argmax: [R][2 n_vt], one entry per tile and wave column
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

// Sixteen zero bytes: the source of every loaded chunk that lies outside the
// operands (rows past R or V, columns past H).
__device__ __attribute__((aligned(16))) const uint4 kLmZero16 = {0u, 0u, 0u, 0u};

// LDS layout of a stage: the hidden rows' chunks, then the unembedding rows'
// chunks, row-major, with the chunk index of row r XORed with lm_swz(r).
// An operand fetch reads one chunk from each of 32 consecutive rows; the
// swizzle spreads any 8 consecutive rows over the 32 banks of 128 bytes and
// any 16 over 64 banks of 256 bytes (both bank widths are conflict-free).
__device__ __forceinline__ int lm_swz(int r) {
    return ((((r >> 2) ^ (r >> 3)) & 1) << 1) | (((r >> 1) ^ (r >> 2)) & 1);
}

// Wait until at most N of this wave's vector-memory operations are
// outstanding (direct-to-LDS loads count here) and its LDS reads are done,
// then meet the workgroup.  A plain s_barrier, not __syncthreads: the
// latter's release fence would wait for every load in flight.
template <int N>
__device__ __forceinline__ void lm_wait_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (0x7 << 4) | (0x0 << 8));
    __builtin_amdgcn_s_barrier();
}

// Schedule.  Workgroup g serves XCD x = g % 8 as its member j = g / 8 of
// GX = grid / 8: workgroups are dispatched to the 8 XCDs in turn (each XCD
// with its own L2), so this keeps the row tiles of a vocabulary tile, which
// read the same unembedding rows, on one XCD at about the same time.  XCD x
// owns the vocabulary tiles vt = x, x + 8, ... and, for each, the n_rt row
// tiles: its list of n_x tiles u = (vt / 8) n_rt + rt, of which member j
// takes j, j + GX, ...; the tiles of a last partial round are cut into
// half tiles when that keeps more members busy (below).  (Cutting them along
// the hidden dimension instead was measured slower: the fp32 partial sums
// the pieces must exchange through agent-scope memory cost more than the
// idle members.)  Only the speed, not the result, depends on where the
// workgroups run.
template <int EPI>
__global__ void __launch_bounds__(kLmThreads, kLmPerCU) k_lmhead(LmArgs a) {
    // the ring stages are separate LDS objects, each named statically where
    // it is used: the compiler then sees that a stage being read is not one
    // that a load in flight writes, and adds no wait for those loads
    __shared__ __attribute__((aligned(16))) uint4 sT0[kLmStage];
    __shared__ __attribute__((aligned(16))) uint4 sT1[kLmStage];
    __shared__ __attribute__((aligned(16))) uint4 sT2[kLmStage];
    __shared__ __attribute__((aligned(16))) uint4 sT3[kLmStage];
    static_assert(kLmStages == 4, "the ring is sT0 .. sT3");
    __shared__ LmPart sP[kLmM][kLmWN];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wm = wave / kLmWN, wn = wave % kLmWN;
    const int n_steps = (a.H + kLmK - 1) / kLmK;
    // operand fetch: per-lane chunk offsets of the two 16-wide slices of a step
    const int fr = lane & 31, fsw = lm_swz(fr);
    const int fc0 = (0 + (lane >> 5)) ^ fsw, fc1 = (2 + (lane >> 5)) ^ fsw;
    const int fw0 = kLmStageA + (wn * (kLmNI * 32) + fr) * kLmChunks;
    const int x = blockIdx.x & 7, j = blockIdx.x >> 3, GX = gridDim.x >> 3;
    const int n_x = (x < a.n_vt ? (a.n_vt - x + 7) / 8 : 0) * a.n_rt;

    lm_float16 acc[kLmMI][kLmNI];

    // acc = the product of rows [r0, r0 + height) of row tile rt and the
    // tokens of vocabulary tile vt; height = kLmM, or kLmM / 2 for a half
    // tile (HALF: only that many hidden rows are loaded, and each wave keeps
    // one 32-row block).
    auto run = [&](auto half_c, int rt, int vt, int r0) {
        constexpr bool HALF = decltype(half_c)::value;
        constexpr int MI = HALF ? 1 : kLmMI;             // 32-row blocks per wave
        constexpr int DA = MI * 32 * kLmWM * kLmChunks / kLmThreads;  // hidden loads per thread and step
        const int row0 = rt * kLmM + r0, v0 = vt * kLmN;
        const int fa0 = (wm * (MI * 32) + fr) * kLmChunks;
#pragma unroll
        for (int mi = 0; mi < MI; ++mi)
#pragma unroll
            for (int ni = 0; ni < kLmNI; ++ni)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[mi][ni][i] = 0.f;
        // The hidden dimension is walked from a step that depends on the
        // vocabulary tile: the row pitch is usually a large power of two, so
        // tiles walking in lockstep would all read the same L2 channels.  The
        // order depends on the token alone, so the logits of a token are the
        // same whatever the rows, the tiling or the epilogue.
        const int rot = (int)(((unsigned)vt * 37u) % (unsigned)n_steps);
        // The loop over the steps, for a wave that issues DW unembedding
        // loads per step (the 64-chunk blocks of a step do not split evenly
        // over the waves, and each wave must wait for exactly its own).
        auto body = [&](auto dw_c) {
            constexpr int DW = decltype(dw_c)::value;
            constexpr int DMA = DA + DW;
            // Direct loads: hidden load q of wave w fills block b = 8 q + w
            // of the hidden region, unembedding load q block 8 q + w of the
            // unembedding region; lane l takes chunk position 64 b + l, i.e.
            // row p / 4 and logical chunk (p % 4) ^ lm_swz(row).  A chunk
            // outside the operands comes from kLmZero16.
            const uint16_t* src[DMA];
            int col[DMA];
#pragma unroll
            for (int q = 0; q < DMA; ++q) {
                const bool isA = q < DA;
                const int b = (isA ? q : q - DA) * kLmWaves + wave, p = b * 64 + lane;
                const int r = p / kLmChunks;
                col[q] = ((p % kLmChunks) ^ lm_swz(r)) * 8;
                if (isA) {
                    const int g = row0 + r;
                    src[q] = g >= a.R ? nullptr : g < a.R1 ? a.hidden + (size_t)g * a.H : a.hidden2 + (size_t)(g - a.R1) * a.H;
                } else {
                    const int g = v0 + r;
                    src[q] = g >= a.V ? nullptr : a.w + (size_t)g * a.H;
                }
            }
            auto issue = [&](int s, uint4* base) {
                const int h0 = s < n_steps ? ((s + rot) % n_steps) * kLmK : a.H;  // past the last step: zeros
#pragma unroll
                for (int q = 0; q < DMA; ++q) {
                    const bool isA = q < DA;
                    const int b = (isA ? q : q - DA) * kLmWaves + wave;
                    const int h = h0 + col[q];
                    const void* g = (src[q] != nullptr && h < a.H) ? (const void*)(src[q] + h) : (const void*)&kLmZero16;
                    __builtin_amdgcn_global_load_lds(g, (lm_lds_void*)(base + (isA ? 0 : kLmStageA) + b * 64), 16, 0, 0);
                }
            };
            auto compute = [&](const uint4* st) {
#pragma unroll
                for (int ks = 0; ks < kLmK / 16; ++ks) {
                    const int fc = ks == 0 ? fc0 : fc1;
                    lm_bf16x8 fa[MI], fb[kLmNI];
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
                        fa[mi] = __builtin_bit_cast(lm_bf16x8, st[fa0 + mi * 32 * kLmChunks + fc]);
#pragma unroll
                    for (int ni = 0; ni < kLmNI; ++ni)
                        fb[ni] = __builtin_bit_cast(lm_bf16x8, st[fw0 + ni * 32 * kLmChunks + fc]);
#pragma unroll
                    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                        for (int ni = 0; ni < kLmNI; ++ni)
                            acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
                }
            };
            // Step s multiplies stage s % 4.  Before it, each wave waits for
            // its own loads of step s (those of steps s + 1 and s + 2 stay in
            // flight) and the barrier makes every wave's loads visible; it
            // also shows that every wave has finished step s - 1, whose stage
            // then takes the loads of step s + 3.  Steps run in fours so that
            // each stage is named statically, and the loop has one exit, at
            // its bottom: the steps past the last (at most three) load zeros
            // and add nothing.
            auto step = [&](int s, const uint4* rd, uint4* wr) {
                lm_wait_barrier<2 * DMA>();
                issue(s + 3, wr);
                compute(rd);
            };
            issue(0, sT0);
            issue(1, sT1);
            issue(2, sT2);
            for (int s = 0; s < n_steps; s += 4) {
                step(s, sT0, sT3);
                step(s + 1, sT1, sT0);
                step(s + 2, sT2, sT1);
                step(s + 3, sT3, sT2);
            }
            // Before the ring is refilled: every wave is done reading it and
            // this wave's loads (and stores) have drained.
            lm_wait_barrier<0>();
        };
        // waves [0, kLmBlkW % 8) take one unembedding block more than the rest
        if constexpr (kLmBlkW % kLmWaves == 0) {
            body(std::integral_constant<int, kLmBlkW / kLmWaves>());
        } else {
            if (wave < kLmBlkW % kLmWaves)
                body(std::integral_constant<int, kLmBlkW / kLmWaves + 1>());
            else
                body(std::integral_constant<int, kLmBlkW / kLmWaves>());
        }
    };

    // The epilogue of run(half, rt, vt, r0).  The argmax parts are kept per
    // wave column: entry 2 vt + c of a row covers tokens
    // [vt kLmN + c kLmN / 2, + kLmN / 2).
    auto epilogue = [&](auto half_c, int rt, int vt, int r0) {
        constexpr bool HALF = decltype(half_c)::value;
        constexpr int MI = HALF ? 1 : kLmMI;
        constexpr int RT = MI * 32 * kLmWM;  // rows of this tile
        const int row0 = rt * kLmM + r0, v0 = vt * kLmN;
        if constexpr (EPI == LM_STORE) {
            // bf16 logits: lanes of a half-wave hold 32 consecutive tokens of one row
#pragma unroll
            for (int mi = 0; mi < MI; ++mi)
#pragma unroll
                for (int ni = 0; ni < kLmNI; ++ni)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int r = row0 + wm * (MI * 32) + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                        const int n = v0 + wn * (kLmNI * 32) + ni * 32 + (lane & 31);
                        if (r < a.R && n < a.V) a.logits[(size_t)r * a.V + n] = lm_bf16_rne(acc[mi][ni][i]);
                    }
        } else {
            // per row of this wave's block: the best over its tokens (the
            // column blocks, then the 32 lanes of the half-wave holding the row)
#pragma unroll
            for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int n0 = v0 + wn * (kLmNI * 32) + (lane & 31);
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
                        sP[wm * (MI * 32) + mi * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3)][wn] = LmPart{bv, bi};
                }
            }
            __syncthreads();
            static_assert(kLmWN == 2, "two parts per row and tile");
            for (int r = tid; r < RT; r += kLmThreads) {
                if (row0 + r >= a.R) break;
                LmPart* out = a.part + (size_t)(row0 + r) * (2 * a.n_vt) + 2 * vt;
                out[0] = sP[r][0];
                out[1] = sP[r][1];
            }
            __syncthreads();  // sP is written again by the next tile
        }
    };

    // Whole tiles j, j + GX, ... while whole rounds of GX remain.  The Q
    // tiles left for the last round would keep only Q of the GX members
    // busy; when 2 Q <= GX they are cut into 2 Q half tiles (128 rows), one
    // per member, which costs each of them about three quarters of a tile
    // (the unembedding rows are read whole) instead of idling the rest.  A
    // half tile that holds no row (past R) is skipped.
    const int F = n_x / GX, Q = n_x - F * GX;
    const bool halves = 2 * Q <= GX;
    const int whole = halves ? F * GX : n_x;
    for (int u = j; u < whole; u += GX) {
        const int rt = u % a.n_rt, vt = (u / a.n_rt) * 8 + x;
        run(std::false_type(), rt, vt, 0);
        epilogue(std::false_type(), rt, vt, 0);
    }
    if (halves && j < 2 * Q) {
        const int u = F * GX + (j >> 1), r0 = (j & 1) * (kLmM / 2);
        const int rt = u % a.n_rt, vt = (u / a.n_rt) * 8 + x;
        if (rt * kLmM + r0 < a.R) {
            run(std::true_type(), rt, vt, r0);
            epilogue(std::true_type(), rt, vt, r0);
        }
    }
}

// A row's argmax over its tile parts (thread 0 returns it; 256 threads).
__device__ __forceinline__ int lm_merge_row(const LmArgs& a, int row, float* s_v, int* s_i) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const LmPart* p = a.part + (size_t)row * (2 * a.n_vt);
    float bv = -INFINITY;
    int bi = INT32_MAX;
    for (int t = tid; t < 2 * a.n_vt; t += 256) {
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
    }
    return bi;
}

__global__ void __launch_bounds__(256) k_lmhead_merge(LmArgs a) {
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    const int row = blockIdx.x;
    const int bi = lm_merge_row(a, row, s_v, s_i);
    if (threadIdx.x == 0) a.gidx[row] = bi;
}

// The merge with the greedy prefix match folded in (fewer than kSplitRows
// sequences): the last of a sequence's rows to be merged writes its outputs.
__global__ void __launch_bounds__(256) k_lmhead_merge_greedy(LmArgs a, GreedyArgs g) {
    __shared__ float s_v[4];
    __shared__ int s_i[4];
    __shared__ GreedyShared S;
    const int row = blockIdx.x;
    const int bi = lm_merge_row(a, row, s_v, s_i);
    greedy_arrive(g, row, bi, S);
}

}  // namespace sv
