// tree_kernels.h — token-tree verification ("Speculative decoding and
// multi-token prediction: how LLMs generate faster", section "Multi-head and
// tree speculation": the target model evaluates all branches of a tree of
// proposals in a single forward pass, and verification returns the one root
// path that survives).
//
// A sequence's tree has N nodes; node i carries a token and a parent index,
// -1 (the committed context, the root) or a node below i (any other value
// leaves the node unreachable).  Target row 0 of the sequence is the root's
// distribution, row i+1 the distribution after node i.  The children of a
// node are proposals made with certainty, so each is a point-mass draft:
//
//  k_tree_walk   : sampling.  From the root, the children of the current
//                  node are tested in index order, child c accepted when
//                  u_c < p(x_c) with p renormalised after each rejected
//                  sibling's token is removed, i.e. u_c * R < p(x_c) with R
//                  the mass left.  A sibling repeating an earlier sibling's
//                  token has nothing left to accept.  The walk records the
//                  path, the row where it stopped and the stop node's child
//                  tokens; the draw kernels then draw from that row with
//                  those tokens removed (a leaf: the bonus draw).
//  k_tree_greedy : temperature 0.  Follow the first child whose token is
//                  the argmax of the current row, then emit that argmax.
//
// One wave per sequence: the node data sits in LDS and each level of the
// walk is a few ballots over the node list, so no step waits on memory.
#pragma once

#include "seq_kernels.h"

namespace sv {

constexpr int kTreeMax = 1024;  // nodes per tree

struct TreeArgs {
    Shape sh;              // target rows [B][N+1][V] (K = N, no per-row tokens)
    const int32_t* tok;    // [B][N] node tokens
    const int32_t* par;    // [B][N] parent indices
    double inv_T;
    uint64_t seed;
    const RowRec* rec;     // sampling: row records (maximum, threshold, kept mass)
    const int32_t* gidx;   // greedy: argmax of every row
    TreeStop* tstop;       // sampling: where each walk stopped
    int32_t* tex;          // sampling: [B][N] child tokens of the stop node
    int32_t* out_tokens;   // [B][N+1]
    int32_t* out_num;      // [B]
    int32_t* out_path;     // [B][N], or null
};

// Path outputs of one sequence: the path's tokens, then (greedy) the last
// token, then -1; the node indices of the path, then -1.  A sampling walk
// leaves the last token's place to the draw.
__device__ __forceinline__ void tree_write_path(const TreeArgs& a, int b, int depth, const int* s_path,
                                                const int* s_tok, int last) {
    const int N = a.sh.K;
    int32_t* out = a.out_tokens + (size_t)b * (N + 1);
    for (int k = threadIdx.x; k <= N; k += 64) {
        if (k < depth) out[k] = s_tok[s_path[k]];
        else if (k > depth) out[k] = -1;
        else if (last >= 0) out[k] = last;
    }
    if (a.out_path)
        for (int k = threadIdx.x; k < N; k += 64) a.out_path[(size_t)b * N + k] = k < depth ? s_path[k] : -1;
    if (threadIdx.x == 0) a.out_num[b] = depth;
}

__global__ void __launch_bounds__(64) k_tree_walk(TreeArgs a) {
    __shared__ int s_par[kTreeMax], s_tok[kTreeMax], s_ex[kTreeMax], s_path[kTreeMax];
    __shared__ double s_p[kTreeMax];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int N = a.sh.K, V = a.sh.V;
    const int32_t* par = a.par + (size_t)b * N;
    const int32_t* tok = a.tok + (size_t)b * N;
    // p of each node's token under its parent's processed row
    for (int i = lane; i < N; i += 64) {
        const int pi = par[i], x = tok[i];
        s_par[i] = pi;
        s_tok[i] = x;
        double p = 0.0;
        if (pi >= -1 && pi < i && x >= 0 && x < V) {
            const int r = b * (N + 1) + pi + 1;
            const spec_row_stats_t& R = a.rec[r].s;
            const float xv = load_logit(row_ptr(a.sh, r), a.sh.tdt, x);
            if (xv >= R.thresh) p = exp(((double)xv - (double)R.max_logit) * a.inv_T) / R.z_kept;
        }
        s_p[i] = p;
    }
    __syncthreads();
    const unsigned long long below = (1ull << lane) - 1ull;
    int u = -1, depth = 0, n_ex = 0;
    for (;;) {
        double R = 1.0;  // mass of p left after the rejected siblings
        int next = -1;
        n_ex = 0;
        // children have indices above their parent
        for (int i0 = u + 1; i0 < N; i0 += 64) {
            const int i = i0 + lane;
            const bool ch = i < N && s_par[i] == u;
            const unsigned long long m = __ballot(ch);
            if (!m) continue;
            const int x = ch ? s_tok[i] : -1;
            // an earlier sibling with the same token: earlier chunks, then
            // lower lanes of this one
            bool dup = false;
            for (int e = 0; e < n_ex; ++e) dup |= s_ex[e] == x;
            for (unsigned long long mm = m; mm; mm &= mm - 1ull) {
                const int l = __ffsll((long long)mm) - 1;
                // every lane takes part in the shuffle: a read from a lane
                // that is not active returns 0, which would match token 0
                const int xl = __shfl(x, l);
                dup |= l < lane && xl == x;
            }
            const bool live = ch && !dup;
            const double pv = live ? s_p[i] : 0.0;
            const double incl = wave_incl_scan(pv);
            const double excl = wave_shift_up1(incl);
            const double ua = ch ? uniform24(draw_block(a.seed, (uint32_t)b, (uint32_t)i, PURPOSE_ACCEPT)) : 1.0;
            const unsigned long long am = __ballot(live && ua * (R - excl) < pv);
            if (ch) s_ex[n_ex + __popcll(m & below)] = x;
            n_ex += __popcll(m);
            __syncthreads();
            if (am) {
                next = i0 + __ffsll((long long)am) - 1;
                break;
            }
            R -= __shfl(incl, 63);
        }
        if (next < 0) break;
        if (lane == 0) s_path[depth] = next;
        ++depth;
        u = next;
    }
    __syncthreads();
    for (int e = lane; e < n_ex; e += 64) a.tex[(size_t)b * N + e] = s_ex[e];
    if (lane == 0) a.tstop[b] = TreeStop{u + 1, depth, n_ex, 0};
    tree_write_path(a, b, depth, s_path, s_tok, -1);
}

__global__ void __launch_bounds__(64) k_tree_greedy(TreeArgs a) {
    __shared__ int s_par[kTreeMax], s_tok[kTreeMax], s_g[kTreeMax + 1], s_path[kTreeMax];
    const int b = blockIdx.x, lane = threadIdx.x;
    const int N = a.sh.K;
    for (int i = lane; i < N; i += 64) {
        s_par[i] = a.par[(size_t)b * N + i];
        s_tok[i] = a.tok[(size_t)b * N + i];
    }
    for (int r = lane; r <= N; r += 64) s_g[r] = a.gidx[(size_t)b * (N + 1) + r];
    __syncthreads();
    int u = -1, depth = 0;
    for (;;) {
        const int g = s_g[u + 1];
        int next = -1;
        for (int i0 = u + 1; i0 < N; i0 += 64) {
            const int i = i0 + lane;
            const unsigned long long m = __ballot(i < N && s_par[i] == u && s_tok[i] == g);
            if (m) {
                next = i0 + __ffsll((long long)m) - 1;
                break;
            }
        }
        if (next < 0) break;
        if (lane == 0) s_path[depth] = next;
        ++depth;
        u = next;
    }
    __syncthreads();
    tree_write_path(a, b, depth, s_path, s_tok, s_g[u + 1]);
}

}  // namespace sv
