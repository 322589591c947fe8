// seq_kernels.h — per-sequence kernels: the accept scan over K drafted
// positions and the draw of the stop token.
//
//  k_seq_filtered : filtered rows (top-k / top-p).  p_j is nonzero only on the
//                   stop target row's kept set, stored sorted by index by
//                   k_row, so the residual max(0, p_j - q_j) is evaluated on
//                   that list (with the draft logits stored beside it).  One
//                   workgroup per (sequence, possible stop position).
//  k_draw : unfiltered rows.  The residual is spread over the whole
//                   vocabulary: one workgroup per (sequence, chunk) sums the
//                   stop row pair's fp64 weights, and the last of a
//                   sequence's chunk workgroups to finish takes the exact
//                   normalisers and locates the draw.
//  k_greedy_prefix : greedy prefix match from the per-row argmax.
//
// k_draw also serves token trees (filtered or not): there a
// walk kernel has already fixed each sequence's stop row, the depth of its
// accepted path and the tokens of the stop node's children (all rejected),
// which the draw removes from p_j the way a point-mass draft's token is
// removed.
#pragma once

#include <type_traits>

#include "row_kernels.h"

namespace sv {

constexpr int kSB = 256;                 // threads per sequence workgroup
constexpr int kChunk = 1024;             // tokens per draw chunk
constexpr int kCPT = kChunk / kSB;       // 4 contiguous tokens per thread

// Where the walk of a token tree stopped: the target row of the stop node,
// the number of accepted nodes, and how many children (all rejected) the
// stop node has; none means the draw is the bonus draw from p of that row.
struct TreeStop {
    int row, depth, n_ex, pad;
};

struct DrawChunk;

struct SeqArgs {
    Shape sh;
    double inv_T;
    uint64_t seed;
    const RowRec* rec;
    const uint2* kept;
    const int* kept_n;
    const float* kept_d;  // draft logit of each listed token (stop positions j < K)
    const double* kept_p; // p of each listed token
    DrawChunk* chunks;         // [B][n_chunks] chunk records of the unfiltered draw
    unsigned* draw_cnt;   // [B * kCntStride] arrival counters of the chunk workgroups (zero between calls)
    int n_chunks;
    int32_t* out_tokens;
    int32_t* out_num;
    int point;            // drafts are point masses at the drafted tokens (no draft rows)
    const TreeStop* tstop; // token trees: per-sequence stop (null for drafted sequences)
    const int32_t* tex;    // token trees: [B][K] tokens of the stop node's children
};

// Stop position of sequence b: first k with !(u_k * q_k(d_k) < p_k(d_k)),
// or K.  Executed by one wave; every lane returns it.
__device__ __forceinline__ int first_rejection(const SeqArgs& a, int b) {
    const int lane = threadIdx.x & 63;
    const int K = a.sh.K;
    const int Kb = seq_len(a.sh, b);
    for (int k0 = 0; k0 < Kb; k0 += 64) {
        const int k = k0 + lane;
        bool reject = false;
        if (k < Kb) {
            const double p = a.rec[(size_t)b * (K + 1) + k].s.prob_at_token;
            // a point-mass draft gives its own token probability 1
            const double q = a.point ? 1.0 : a.rec[a.sh.n_trows + (size_t)b * K + k].s.prob_at_token;
            const double u = uniform24(draw_block(a.seed, (uint32_t)b, (uint32_t)k, PURPOSE_ACCEPT));
            reject = !(u * q < p);
        }
        const unsigned long long m = __ballot(reject);
        if (m) return k0 + __ffsll((long long)m) - 1;
    }
    return Kb;
}

// The stop row of sequence b: fixed by the walk for a token tree, else the
// first rejection.  Executed by one wave.  The kernels take the tree case as
// a template parameter, so the drafted-sequence code carries none of it.
template <bool kTree>
__device__ __forceinline__ int stop_of(const SeqArgs& a, int b) {
    if constexpr (kTree) return a.tstop[b].row;
    else return first_rejection(a, b);
}
// The stop row pair of a sequence: target row j, draft row j when j < K_b
// (or, for point-mass drafts, the drafted token dtok, where q = 1).
struct StopRow {
    const char* tp;
    const char* dp;
    int tdt, ddt;
    float Mt, Md, thr_t, thr_d;
    double zt, zd;
    bool has_draft;
    bool bonus;  // j is the sequence's draft length: the bonus row, drawn from p_j
    int dtok;    // -1 unless the draft is a point mass at dtok
    const int32_t* ex;  // token trees: tokens removed from p_j (the rejected children)
    int n_ex;
};


template <bool kTree>
__device__ __forceinline__ StopRow stop_row(const SeqArgs& a, int b, int j) {
    StopRow s;
    const int K = a.sh.K;
    const int rt = b * (K + 1) + j;
    const RowRec& Rt = a.rec[rt];
    s.tp = row_ptr(a.sh, rt);
    s.tdt = a.sh.tdt;
    s.Mt = Rt.s.max_logit;
    s.thr_t = Rt.s.thresh;
    s.zt = Rt.s.z_kept;
    s.n_ex = 0;
    s.ex = nullptr;
    if constexpr (kTree) {
        s.n_ex = a.tstop[b].n_ex;
        s.ex = a.tex + (size_t)b * K;
        s.bonus = s.n_ex == 0;
        s.has_draft = false;
        s.dtok = -1;
    } else {
        const int Kb = seq_len(a.sh, b);
        s.bonus = j >= Kb;
        s.has_draft = j < Kb && !a.point;
        s.dtok = j < Kb && a.point ? a.sh.tokens[(size_t)b * K + j] : -1;
    }
    if (s.has_draft) {
        const int rd = a.sh.n_trows + b * K + j;
        const RowRec& Rd = a.rec[rd];
        s.dp = row_ptr(a.sh, rd);
        s.ddt = a.sh.ddt;
        s.Md = Rd.s.max_logit;
        s.thr_d = Rd.s.thresh;
        s.zd = Rd.s.z_kept;
    } else {
        s.dp = nullptr;
        s.ddt = 0;
        s.Md = 0.f;
        s.thr_d = 0.f;
        s.zd = 1.0;
    }
    return s;
}

// p_j(i) and the residual max(0, p_j(i) - q_j(i)) in fp64, given the target
// logit xt of token i.
__device__ __forceinline__ void stop_terms_x(const StopRow& s, double inv_T, int i, float xt,
                                             double& p, double& r) {
    p = xt >= s.thr_t ? exp(((double)xt - (double)s.Mt) * inv_T) / s.zt : 0.0;
    double q = i == s.dtok ? 1.0 : 0.0;
    if (s.has_draft) {
        const float xd = load_logit(s.dp, s.ddt, i);
        q = xd >= s.thr_d ? exp(((double)xd - (double)s.Md) * inv_T) / s.zd : 0.0;
    }
    const double d = p - q;
    r = d > 0.0 ? d : 0.0;
}
__device__ __forceinline__ void stop_terms(const StopRow& s, double inv_T, int i, double& p, double& r) {
    stop_terms_x(s, inv_T, i, load_logit(s.tp, s.tdt, i), p, r);
}

// Deterministic exclusive scan of one double per thread (thread order) over
// kSB threads; also returns the total.  The same code produces chunk totals
// and search prefixes, so both see identical values.
__device__ __forceinline__ void seq_excl_scan(double v, double* s_val, double* s_excl, double* s_total, double& excl,
                              double& total) {
    const int tid = threadIdx.x;
    s_val[tid] = v;
    __syncthreads();
    if (tid < 64) {
        const double v0 = s_val[4 * tid], v1 = s_val[4 * tid + 1];
        const double v2 = s_val[4 * tid + 2], v3 = s_val[4 * tid + 3];
        const double ls = ((v0 + v1) + v2) + v3;
        const double incl = wave_incl_scan(ls);
        double e = wave_shift_up1(incl);
        s_excl[4 * tid] = e;
        e += v0;
        s_excl[4 * tid + 1] = e;
        e += v1;
        s_excl[4 * tid + 2] = e;
        e += v2;
        s_excl[4 * tid + 3] = e;
        if (tid == 63) *s_total = incl;
    }
    __syncthreads();
    excl = s_excl[tid];
    total = *s_total;
    __syncthreads();
}

// The thread whose range holds the draw point t: the last thread with
// positive mass whose range starts at or before t (or, if rounding put t
// before every positive range, the first one with positive mass).
__device__ __forceinline__ int pick_thread(double mine, double run_excl, double t, int* s_tau) {
    if (threadIdx.x == 0) *s_tau = -1;
    __syncthreads();
    if (mine > 0.0 && run_excl <= t) atomicMax(s_tau, (int)threadIdx.x);
    __syncthreads();
    int tau = *s_tau;
    if (tau < 0) {
        __syncthreads();
        if (threadIdx.x == 0) *s_tau = kSB;
        __syncthreads();
        if (mine > 0.0) atomicMin(s_tau, (int)threadIdx.x);
        __syncthreads();
        tau = *s_tau;
    }
    __syncthreads();
    return tau;
}

// Per-position acceptance counters of sequence b (num_accepted j): its test
// at position k ran for k <= j, k < K_b, and accepted for k < j.  Integer
// atomics, so the totals do not depend on order.
__device__ __forceinline__ void count_accepts(const Shape& sh, int b, int j) {
    if (sh.tested) {
        const int nt = min(j + 1, seq_len(sh, b));
        for (int k = 0; k < nt; ++k) atomicAdd(&sh.tested[k], 1);
    }
    if (sh.accepted)
        for (int k = 0; k < j; ++k) atomicAdd(&sh.accepted[k], 1);
}

template <bool kTree>
__device__ __forceinline__ void write_outputs(const SeqArgs& a, int b, int j, int y) {
    const int K = a.sh.K;
    if constexpr (kTree) {  // the walk wrote the path, the count and the padding
        a.out_tokens[(size_t)b * (K + 1) + a.tstop[b].depth] = y;
        return;
    }
    int32_t* out = a.out_tokens + (size_t)b * (K + 1);
    for (int k = 0; k < j; ++k) out[k] = a.sh.tokens[(size_t)b * K + k];
    out[j] = y;
    for (int k = j + 1; k <= K; ++k) out[k] = -1;
    a.out_num[b] = j;
    count_accepts(a.sh, b, j);
}

// Draw over the whole stop row pair with one workgroup (thread-contiguous
// token ranges).  Used when no kept list is available.
__device__ __forceinline__ void draw_full_row(const SeqArgs& a, int b, int j, double* s_val, double* s_excl,
                              double* s_total, int* s_tau) {
    const StopRow s = stop_row<false>(a, b, j);
    const int V = a.sh.V;
    const int per = (V + kSB - 1) / kSB;
    const int lo = threadIdx.x * per, hi = min(lo + per, V);
    double sr = 0.0, sp = 0.0;
    for (int i = lo; i < hi; ++i) {
        double p, r;
        stop_terms(s, a.inv_T, i, p, r);
        sr += r;
        sp += p;
    }
    double er, tr, ep, tp;
    seq_excl_scan(sr, s_val, s_excl, s_total, er, tr);
    seq_excl_scan(sp, s_val, s_excl, s_total, ep, tp);
    const bool usep = s.bonus || !(tr > 0.0);
    const double S = usep ? tp : tr;
    const double t = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)j, PURPOSE_SAMPLE)) * S;
    const double mine = usep ? sp : sr;
    const double ex = usep ? ep : er;
    const int tau = pick_thread(mine, ex, t, s_tau);
    if ((int)threadIdx.x == tau) {
        double acc = ex;
        int y = -1, last = -1;
        for (int i = lo; i < hi; ++i) {
            double p, r;
            stop_terms(s, a.inv_T, i, p, r);
            const double w = usep ? p : r;
            if (w > 0.0) {
                last = i;
                acc += w;
                if (acc > t) {
                    y = i;
                    break;
                }
            }
        }
        write_outputs<false>(a, b, j, y >= 0 ? y : last);
    }
}

// Draw over a kept list longer than the speculative load: thread-contiguous
// slices of up to kListMax / kSB entries, read and gathered now.
constexpr int kListPT = kListMax / kSB;  // 16

__device__ __forceinline__ void draw_long_list(const SeqArgs& a, int b, int j, int n, const uint2* L,
                                               const StopRow& s, double* s_val, double* s_excl,
                                               double* s_total, int* s_tau) {
    const int per = (n + kSB - 1) / kSB;
    const int lo = threadIdx.x * per, hi = min(lo + per, n);
    double pr[kListPT], rr[kListPT];
    int ix[kListPT];
    double sr = 0.0, sp = 0.0;
#pragma unroll
    for (int e = 0; e < kListPT; ++e) {
        pr[e] = 0.0;
        rr[e] = 0.0;
        ix[e] = -1;
        const int i = lo + e;
        if (e < per && i < hi) {
            const uint2 ent = L[i];
            ix[e] = (int)ent.x;
            stop_terms_x(s, a.inv_T, (int)ent.x, __uint_as_float(ent.y), pr[e], rr[e]);
            sr += rr[e];
            sp += pr[e];
        }
    }
    double er, tr, ep, tp;
    seq_excl_scan(sr, s_val, s_excl, s_total, er, tr);
    seq_excl_scan(sp, s_val, s_excl, s_total, ep, tp);
    const bool usep = s.bonus || !(tr > 0.0);
    const double S = usep ? tp : tr;
    const double t = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)j, PURPOSE_SAMPLE)) * S;
    const double mine = usep ? sp : sr;
    const double ex = usep ? ep : er;
    const int tau = pick_thread(mine, ex, t, s_tau);
    if ((int)threadIdx.x == tau) {
        double acc = ex;
        int y = -1, last = -1;
#pragma unroll
        for (int e = 0; e < kListPT; ++e) {
            const double w = usep ? pr[e] : rr[e];
            if (y < 0 && ix[e] >= 0 && w > 0.0) {
                last = ix[e];
                acc += w;
                if (acc > t) y = ix[e];
            }
        }
        write_outputs<false>(a, b, j, y >= 0 ? y : last);
    }
}

// ---------------------------------------------------------------------------
// Filtered: one workgroup per (sequence, candidate stop position j).  Every
// workgroup loads, in one round, the accept-test inputs of its sequence, the
// records of row pair j and the first kSpec entries of target row j's kept
// list with the p values and draft logits the row kernel stored beside them; the
// workgroup whose j is the stop position then draws, the others exit.  So
// one dependent memory round separates the row kernel from the output.
// ---------------------------------------------------------------------------
constexpr int kLPT = 4;                  // kept-list entries per thread
constexpr int kSpec = kLPT * kSB;        // entries loaded before the stop is known (1024)

// Exclusive prefix sums of two doubles over the kSB threads in thread order
// (wave scans, then the wave totals), and their totals.
__device__ __forceinline__ void seq_excl_scan2(double a, double b, double* s_wa, double* s_wb, double& ea,
                                               double& eb, double& ta, double& tb) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double ia = wave_incl_scan(a), ib = wave_incl_scan(b);
    const double xa = wave_shift_up1(ia), xb = wave_shift_up1(ib);
    if (lane == 63) {
        s_wa[wave] = ia;
        s_wb[wave] = ib;
    }
    __syncthreads();
    double pa = 0.0, pb = 0.0;
    ta = 0.0;
    tb = 0.0;
#pragma unroll
    for (int w = 0; w < kSB / 64; ++w) {
        if (w < wave) {
            pa += s_wa[w];
            pb += s_wb[w];
        }
        ta += s_wa[w];
        tb += s_wb[w];
    }
    ea = pa + xa;
    eb = pb + xb;
}

__global__ void __launch_bounds__(kSB) k_seq_filtered(SeqArgs a) {
    __shared__ double s_val[kSB], s_excl[kSB], s_total;
    __shared__ double s_wa[kSB / 64], s_wb[kSB / 64];
    __shared__ int s_j, s_tau, s_y;
    __shared__ int s_last[kSB / 64], s_first[kSB / 64];
    const int K = a.sh.K;
    const int b = blockIdx.x / (K + 1), jc = blockIdx.x % (K + 1);
    const int rt = b * (K + 1) + jc;
    const int n = a.kept_n[rt];
    const uint2* L = a.kept + (size_t)rt * kListMax;
    // thread-contiguous slices, so thread order is token order
    uint2 ent[kLPT];
#pragma unroll
    for (int e = 0; e < kLPT; ++e) ent[e] = L[threadIdx.x * kLPT + e];
    // p and the draft logits of the listed tokens, stored beside the list by
    // the row kernel (draft logits for positions j < K)
    float xdl[kLPT];
    double pl[kLPT];
    {
        const float* LD = a.kept_d + (size_t)rt * kListMax;
        const double* LP = a.kept_p + (size_t)rt * kListMax;
#pragma unroll
        for (int e = 0; e < kLPT; ++e) {
            xdl[e] = LD[threadIdx.x * kLPT + e];
            pl[e] = LP[threadIdx.x * kLPT + e];
        }
    }
    const StopRow s = stop_row<false>(a, b, jc);
    // the accepted drafted tokens, one per thread, for the output row
    const int tok = (int)threadIdx.x < jc ? a.sh.tokens[(size_t)b * K + threadIdx.x] : -1;
    if (threadIdx.x < 64) {
        const int j = first_rejection(a, b);
        if (threadIdx.x == 0) s_j = j;
    }
    __syncthreads();
    if (s_j != jc) return;
    if (n < 0) {
        draw_full_row(a, b, jc, s_val, s_excl, &s_total, &s_tau);
        return;
    }
    if (n > kSpec) {
        draw_long_list(a, b, jc, n, L, s, s_val, s_excl, &s_total, &s_tau);
        return;
    }
    const double inv_zd = 1.0 / s.zd;
    double pr[kLPT], rr[kLPT];
    double sr = 0.0, sp = 0.0;
#pragma unroll
    for (int e = 0; e < kLPT; ++e) {
        pr[e] = threadIdx.x * kLPT + e < n ? pl[e] : 0.0;
        sp += pr[e];
    }
#pragma unroll
    for (int e = 0; e < kLPT; ++e) {
        const float xd = s.has_draft ? xdl[e] : -INFINITY;
        const bool in = threadIdx.x * kLPT + e < n;
        const bool qd = in && xd >= s.thr_d;
        const double q = qd ? exp(((double)xd - (double)s.Md) * a.inv_T) * inv_zd
                            : (in && (int)ent[e].x == s.dtok ? 1.0 : 0.0);
        const double d = pr[e] - q;
        rr[e] = d > 0.0 ? d : 0.0;
        sr += rr[e];
    }
    double er, ep, tr, tp;
    seq_excl_scan2(sr, sp, s_wa, s_wb, er, ep, tr, tp);
    const bool usep = s.bonus || !(tr > 0.0);
    const double S = usep ? tp : tr;
    const double t = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)jc, PURPOSE_SAMPLE)) * S;
    const double mine = usep ? sp : sr;
    const double ex = usep ? ep : er;
    // the thread whose range holds t: the last one with mass whose range
    // starts at or before t (prefixes are non-decreasing in thread order);
    // if rounding put t before all of them, the first one with mass
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long mc = __ballot(mine > 0.0 && ex <= t);
    const unsigned long long mf = __ballot(mine > 0.0);
    if (lane == 0) {
        s_last[wave] = mc ? wave * 64 + 63 - __clzll((long long)mc) : -1;
        s_first[wave] = mf ? wave * 64 + __ffsll((long long)mf) - 1 : kSB;
    }
    __syncthreads();
    int tau = -1, first = kSB;
#pragma unroll
    for (int w = 0; w < kSB / 64; ++w) {
        tau = max(tau, s_last[w]);
        first = min(first, s_first[w]);
    }
    if (tau < 0) tau = first;
    if ((int)threadIdx.x == tau) {
        double acc = ex;
        int y = -1, last = -1;
#pragma unroll
        for (int e = 0; e < kLPT; ++e) {
            const int i = threadIdx.x * kLPT + e;
            const double w = usep ? pr[e] : rr[e];
            if (y < 0 && i < n && w > 0.0) {
                last = (int)ent[e].x;
                acc += w;
                if (acc > t) y = (int)ent[e].x;
            }
        }
        s_y = y >= 0 ? y : last;
    }
    __syncthreads();
    // output row: accepted drafts, the drawn token, then -1
    int32_t* out = a.out_tokens + (size_t)b * (K + 1);
    for (int k = threadIdx.x; k <= K; k += kSB)
        out[k] = k < jc ? (k < kSB ? tok : a.sh.tokens[(size_t)b * K + k]) : (k == jc ? s_y : -1);
    if (threadIdx.x == 0) {
        a.out_num[b] = jc;
        count_accepts(a.sh, b, jc);
    }
}

// ---------------------------------------------------------------------------
// Unfiltered rows and token trees: the draw over the whole stop row pair.
//
// p_j = e_t / Z_t and q_j = e_d / Z_d with e = exp((x - M) / T) in fp64 and
// Z the fp64 sum of the kept e over the row, so the residual scaled by Z_t is
// max(0, e_t - rho e_d), rho = Z_t / Z_d: the draw depends on rho alone.  The
// exact rho is known only once every chunk of the row pair is summed; the
// row records give an estimate rho~ (fp32 streamed sums, relative error far
// below kDelta / 2).  Each chunk workgroup sums e_t and e_d over its tokens
// and, over the tokens whose residual has the same sign for every rho within
// kDelta / 2 of rho~, the e_t and e_d of the positive ones (their residual
// mass is then a - rho b for any such rho); the few other tokens are listed
// with their weights.  The last chunk workgroup of a sequence to finish takes
// the exact rho, the residual mass of every chunk, the chunk holding the draw
// point and the token inside it.  If rho lies outside the band, or a chunk
// holds more unsettled tokens than it lists, every chunk is recomputed with
// the exact rho (slow, exact).  Point-mass drafts, token trees and the bonus
// row have no draft row: their residual is e_t without the removed tokens.
// ---------------------------------------------------------------------------
constexpr double kDelta = 0x1p-14;
constexpr int kAmb = 8;

struct DrawChunk {
    double zt, zd;              // sums of e_t and e_d over the chunk
    double a, b;                // sums of e_t and e_d over its settled positive tokens
    double at[kAmb], ad[kAmb];  // e_t and e_d of the unsettled tokens, in token order
    int n_amb;                  // unsettled tokens (more than kAmb: not all listed)
    int pad;
};

// The kCPT logits of row `row` from token lo on (-inf past V): the loads of
// a thread are issued together and decoded after.
template <int DT>
__device__ __forceinline__ void load_run(const char* row, int lo, int V, float (&x)[kCPT]) {
    uint32_t raw[kCPT];
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
        const int i = min(lo + e, V - 1);
        raw[e] = DT == DT_F32 ? reinterpret_cast<const uint32_t*>(row)[i]
                              : (uint32_t)reinterpret_cast<const uint16_t*>(row)[i];
    }
#pragma unroll
    for (int e = 0; e < kCPT; ++e)
        x[e] = lo + e < V ? __uint_as_float(DT == DT_F32 ? raw[e] : raw[e] << 16) : -INFINITY;
}

// fp64 weights of the kCPT tokens from lo on: e_t (0 where the target row
// does not keep the token) and e_d (0 without a draft row or where it does
// not keep it).  The same arithmetic wherever a chunk is summed or searched.
template <int TDT, int DDT>
__device__ __forceinline__ void run_weights(const StopRow& s, double inv_T, int lo, int V, double (&et)[kCPT],
                                            double (&ed)[kCPT]) {
    float xt[kCPT], xd[kCPT];
    load_run<TDT>(s.tp, lo, V, xt);
    // without a draft row the target row is read again and ignored
    load_run<DDT>(s.has_draft ? s.dp : s.tp, lo, V, xd);
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
        et[e] = xt[e] >= s.thr_t ? exp(((double)xt[e] - (double)s.Mt) * inv_T) : 0.0;
        ed[e] = (s.has_draft && xd[e] >= s.thr_d) ? exp(((double)xd[e] - (double)s.Md) * inv_T) : 0.0;
    }
}

// Calls f(integral_constant TDT, integral_constant DDT) for the row pair's
// dtypes (uniform over the workgroup).
template <class F>
__device__ __forceinline__ void with_dtypes(const StopRow& s, F&& f) {
    const int ddt = s.has_draft ? s.ddt : s.tdt;
    if (s.tdt == DT_F32) {
        if (ddt == DT_F32) f(std::integral_constant<int, DT_F32>(), std::integral_constant<int, DT_F32>());
        else f(std::integral_constant<int, DT_F32>(), std::integral_constant<int, DT_BF16>());
    } else {
        if (ddt == DT_F32) f(std::integral_constant<int, DT_BF16>(), std::integral_constant<int, DT_F32>());
        else f(std::integral_constant<int, DT_BF16>(), std::integral_constant<int, DT_BF16>());
    }
}

// Residual weight of one token, scaled by Z_t: max(0, e_t - rho e_d) with a
// draft row, else e_t unless the token is removed (where q = 1 >= p).
__device__ __forceinline__ double res_weight(bool has_draft, double et, double ed, bool removed, double rho) {
    if (has_draft) {
        const double d = et - rho * ed;
        return d > 0.0 ? d : 0.0;
    }
    return removed ? 0.0 : et;
}

// Totals of N doubles over the kSB threads (wave butterflies, then the waves
// in order): the same values in every thread.  s[n][w] is scratch; the
// leading barrier lets a previous call's readers finish.
template <int N>
__device__ __forceinline__ void seq_totals(double (&v)[N], double (*s)[kSB / 64]) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = wave_sum(v[n]);
    __syncthreads();
    if (lane == 0)
#pragma unroll
        for (int n = 0; n < N; ++n) s[n][wave] = v[n];
    __syncthreads();
    static_assert(kSB / 64 == 4, "four waves");
#pragma unroll
    for (int n = 0; n < N; ++n) v[n] = (s[n][0] + s[n][1]) + (s[n][2] + s[n][3]);
}

// Exclusive prefix of one int per thread in thread order, and the total.
__device__ __forceinline__ int seq_excl_scan_int(int v, int* s, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) s[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kSB / 64; ++w) {
        before += w < wave ? s[w] : 0;
        total += s[w];
    }
    return before + incl - v;
}

// Loads of another workgroup's chunk records (written with agent-scope
// stores before its arrival was counted): agent-scope, so coherent across the
// GPU's L2 caches.
__device__ __forceinline__ double ld_agent(const double* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(double* p, double v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Waits until this thread's earlier stores are complete (vmcnt 0; the other
// counters left alone).
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Residual mass of one chunk from its record for an exact rho inside the band
// (every listed unsettled token is evaluated; the caller has checked that
// none is missing).
__device__ __forceinline__ double chunk_res(const DrawChunk* c, bool has_draft, double rho) {
    const double a = ld_agent(&c->a);
    if (!has_draft) return a;
    double r = a - rho * ld_agent(&c->b);
    r = r > 0.0 ? r : 0.0;
    const int n = min(ld_agent(&c->n_amb), kAmb);
    for (int k = 0; k < n; ++k) r += res_weight(true, ld_agent(&c->at[k]), ld_agent(&c->ad[k]), false, rho);
    return r;
}

struct DrawShared {
    double tot[4][kSB / 64];
    double run;
    int j, cstar, last, tau;
    int s_last[kSB / 64], s_first[kSB / 64];
    int scan[kSB / 64];
    uint32_t removed[kChunk / 32];  // bitmap of the removed tokens of one chunk
};

// Bit e set: token lo + e (e < kCPT) of chunk cc is removed from p: a token
// tree's rejected children, marked in an LDS bitmap of the chunk (the
// workgroup shares out the list), or a point-mass draft's token.  Called by
// the whole workgroup.
__device__ __forceinline__ uint32_t removed_bits(const StopRow& s, int cc, int lo, DrawShared& S) {
    uint32_t rm = 0u;
    if (s.n_ex > 0) {
        __syncthreads();  // earlier readers of the bitmap are done
        for (int i = threadIdx.x; i < kChunk / 32; i += kSB) S.removed[i] = 0u;
        __syncthreads();
        for (int e = threadIdx.x; e < s.n_ex; e += kSB) {
            const uint32_t d = (uint32_t)(s.ex[e] - cc * kChunk);
            if (d < (uint32_t)kChunk) atomicOr(&S.removed[d >> 5], 1u << (d & 31));
        }
        __syncthreads();
        const int off = lo - cc * kChunk;  // a multiple of kCPT: the kCPT bits share a word
        rm = (S.removed[off >> 5] >> (off & 31)) & ((1u << kCPT) - 1u);
    }
    const uint32_t d = (uint32_t)(s.dtok - lo);
    if (s.dtok >= 0 && d < (uint32_t)kCPT) rm |= 1u << d;
    return rm;
}
static_assert(kChunk % 32 == 0 && 32 % kCPT == 0, "a thread's tokens share a bitmap word");

// The thread whose mass range holds t: the last one with mass starting at or
// before t; if rounding put t before all of them, the first one with mass.
__device__ __forceinline__ int locate_thread(double mine, double ex, double t, DrawShared& S) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const unsigned long long mc = __ballot(mine > 0.0 && ex <= t);
    const unsigned long long mf = __ballot(mine > 0.0);
    __syncthreads();
    if (lane == 0) {
        S.s_last[wave] = mc ? wave * 64 + 63 - __clzll((long long)mc) : -1;
        S.s_first[wave] = mf ? wave * 64 + __ffsll((long long)mf) - 1 : kSB;
    }
    __syncthreads();
    int tau = -1, first = kSB;
#pragma unroll
    for (int w = 0; w < kSB / 64; ++w) {
        tau = max(tau, S.s_last[w]);
        first = min(first, S.s_first[w]);
    }
    return tau >= 0 ? tau : first;
}

// Exclusive prefix (thread order) of one double per thread, and the total.
__device__ __forceinline__ double seq_excl_scan_d(double v, DrawShared& S, double& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const double incl = wave_incl_scan(v);
    const double ex = wave_shift_up1(incl);
    __syncthreads();
    if (lane == 63) S.tot[0][wave] = incl;
    __syncthreads();
    double before = 0.0;
    total = 0.0;
#pragma unroll
    for (int w = 0; w < kSB / 64; ++w) {
        before += w < wave ? S.tot[0][w] : 0.0;
        total += S.tot[0][w];
    }
    return before + ex;
}

// Mass of chunk cc (residual with the exact rho, or p) recomputed by the
// whole workgroup.
template <int TDT, int DDT>
__device__ __forceinline__ double chunk_mass_recomputed(const StopRow& s, double inv_T, int V, int cc, bool usep,
                                                        double rho, DrawShared& S) {
    double et[kCPT], ed[kCPT];
    const uint32_t rm = removed_bits(s, cc, cc * kChunk + (int)threadIdx.x * kCPT, S);
    run_weights<TDT, DDT>(s, inv_T, cc * kChunk + (int)threadIdx.x * kCPT, V, et, ed);
    double m[1] = {0.0};
#pragma unroll
    for (int e = 0; e < kCPT; ++e) m[0] += usep ? et[e] : res_weight(s.has_draft, et[e], ed[e], (rm >> e) & 1u, rho);
    seq_totals<1>(m, S.tot);
    return m[0];
}

// The pick, by the last chunk workgroup of sequence b (stop position j).
template <bool kTree, int TDT, int DDT>
__device__ __forceinline__ void draw_pick(const SeqArgs& a, int b, int j, const StopRow& s, double rt, DrawShared& S) {
    const int n_ch = a.n_chunks, V = a.sh.V;
    const DrawChunk* cs = a.chunks + (size_t)b * n_ch;
    // this thread's chunks are contiguous: [c0, c1)
    const int per = (n_ch + kSB - 1) / kSB;
    const int c0 = min((int)threadIdx.x * per, n_ch), c1 = min(c0 + per, n_ch);
    double v[3] = {0.0, 0.0, 0.0};  // sum e_t, sum e_d, unlisted unsettled tokens
    for (int cc = c0; cc < c1; ++cc) {
        v[0] += ld_agent(&cs[cc].zt);
        v[1] += ld_agent(&cs[cc].zd);
        v[2] += ld_agent(&cs[cc].n_amb) > kAmb ? 1.0 : 0.0;
    }
    seq_totals<3>(v, S.tot);
    const double Zt = v[0];
    const double rho = s.has_draft ? Zt / v[1] : 0.0;
    const bool settled = !s.has_draft || (v[2] == 0.0 && fabs(rho - rt) <= 0.5 * kDelta * rt);
    const double u = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)j, PURPOSE_SAMPLE));
    bool usep;
    double t;
    int cstar;
    double run;
    if (settled) {
        // residual mass of this thread's chunks, then the chunk holding t
        double mr = 0.0, mp = 0.0;
        for (int cc = c0; cc < c1; ++cc) {
            mr += chunk_res(&cs[cc], s.has_draft, rho);
            mp += ld_agent(&cs[cc].zt);
        }
        double tr, tp;
        const double er = seq_excl_scan_d(mr, S, tr);
        const double ep = seq_excl_scan_d(mp, S, tp);
        usep = s.bonus || !(tr > 0.0);
        t = u * (usep ? tp : tr);
        const int tc = locate_thread(usep ? mp : mr, usep ? ep : er, t, S);
        if ((int)threadIdx.x == tc) {
            double r = usep ? ep : er;
            int cs_ = -1, last_nz = c0;
            double run_last = r;
            for (int cc = c0; cc < c1; ++cc) {
                const double sc = usep ? ld_agent(&cs[cc].zt) : chunk_res(&cs[cc], s.has_draft, rho);
                if (sc > 0.0) {
                    if (r + sc > t) {
                        cs_ = cc;
                        break;
                    }
                    last_nz = cc;
                    run_last = r;
                }
                r += sc;
            }
            if (cs_ < 0) {
                cs_ = last_nz;
                r = run_last;
            }
            S.cstar = cs_;
            S.run = r;
        }
        __syncthreads();
        cstar = S.cstar;
        run = S.run;
    } else {
        // every chunk recomputed with the exact rho, in chunk order: the
        // total, then the first chunk whose running sum passes t
        double tr = 0.0;
        for (int cc = 0; cc < n_ch; ++cc) tr += chunk_mass_recomputed<TDT, DDT>(s, a.inv_T, V, cc, false, rho, S);
        usep = s.bonus || !(tr > 0.0);
        t = u * (usep ? Zt : tr);
        run = 0.0;
        cstar = -1;
        int last_nz = 0;
        double run_last = 0.0;
        for (int cc = 0; cc < n_ch; ++cc) {
            const double sc = chunk_mass_recomputed<TDT, DDT>(s, a.inv_T, V, cc, usep, rho, S);
            if (sc > 0.0) {
                if (run + sc > t) {
                    cstar = cc;
                    break;
                }
                last_nz = cc;
                run_last = run;
            }
            run += sc;
        }
        if (cstar < 0) {
            cstar = last_nz;
            run = run_last;
        }
    }
    // the token inside chunk cstar, from the same per-token weights
    const int lo = cstar * kChunk + (int)threadIdx.x * kCPT;
    double et[kCPT], ed[kCPT], w[kCPT];
    const uint32_t rm = removed_bits(s, cstar, lo, S);
    run_weights<TDT, DDT>(s, a.inv_T, lo, V, et, ed);
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
        w[e] = usep ? et[e] : res_weight(s.has_draft, et[e], ed[e], (rm >> e) & 1u, rho);
        mine += w[e];
    }
    double tot;
    const double ex = run + seq_excl_scan_d(mine, S, tot);
    const int tau = locate_thread(mine, ex, t, S);
    if ((int)threadIdx.x == tau) {
        double acc = ex;
        int y = -1, last = -1;
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
            if (y < 0 && w[e] > 0.0) {
                last = lo + e;
                acc += w[e];
                if (acc > t) y = lo + e;
            }
        }
        write_outputs<kTree>(a, b, j, y >= 0 ? y : last);
    }
}

// One workgroup per (sequence, chunk of kChunk tokens): the chunk record of
// the stop row pair, then, in the last of the sequence's chunk workgroups to
// finish, the pick.  The arrival counter of each sequence is zero between
// calls (zeroed with the workspace, reset by the last workgroup).
template <bool kTree>
__global__ void __launch_bounds__(kSB) k_draw(SeqArgs a) {
    __shared__ DrawShared S;
    const int b = blockIdx.x / a.n_chunks;
    const int c = blockIdx.x % a.n_chunks;
    if (threadIdx.x < 64) {
        const int j = stop_of<kTree>(a, b);
        if (threadIdx.x == 0) S.j = j;
    }
    __syncthreads();
    const int j = S.j;
    const StopRow s = stop_row<kTree>(a, b, j);
    // rho~ from the row records
    const double rt = s.has_draft ? s.zt / s.zd : 0.0;
    DrawChunk* rec = a.chunks + (size_t)b * a.n_chunks + c;
    with_dtypes(s, [&](auto tt, auto dt) {
        constexpr int TDT = decltype(tt)::value, DDT = decltype(dt)::value;
        double et[kCPT], ed[kCPT];
        const uint32_t rm = removed_bits(s, c, c * kChunk + (int)threadIdx.x * kCPT, S);
        run_weights<TDT, DDT>(s, a.inv_T, c * kChunk + (int)threadIdx.x * kCPT, a.sh.V, et, ed);
        double v[4] = {0.0, 0.0, 0.0, 0.0};  // zt, zd, a, b
        int amb = 0;                          // this thread's unsettled tokens (bit mask)
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
            v[0] += et[e];
            v[1] += ed[e];
            if (!s.has_draft) {
                v[2] += ((rm >> e) & 1u) ? 0.0 : et[e];
            } else if (ed[e] == 0.0) {
                v[2] += et[e];
            } else {
                const double d = et[e] - rt * ed[e], tol = kDelta * rt * ed[e];
                if (d > tol) {
                    v[2] += et[e];
                    v[3] += ed[e];
                } else if (d >= -tol) {
                    amb |= 1 << e;
                }
            }
        }
        int n_amb;
        int slot = seq_excl_scan_int(__popc(amb), S.scan, n_amb);
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
            if ((amb >> e) & 1) {
                if (slot < kAmb) {
                    st_agent(&rec->at[slot], et[e]);
                    st_agent(&rec->ad[slot], ed[e]);
                }
                ++slot;
            }
        }
        seq_totals<4>(v, S.tot);
        if (threadIdx.x == 0) {
            st_agent(&rec->zt, v[0]);
            st_agent(&rec->zd, v[1]);
            st_agent(&rec->a, v[2]);
            st_agent(&rec->b, v[3]);
            st_agent(&rec->n_amb, n_amb);
        }
    });
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
        S.last = __hip_atomic_fetch_add(&a.draw_cnt[(size_t)b * kCntStride], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                 (unsigned)(a.n_chunks - 1);
    __syncthreads();
    if (!S.last) return;
    with_dtypes(s, [&](auto tt, auto dt) {
        draw_pick<kTree, decltype(tt)::value, decltype(dt)::value>(a, b, j, s, rt, S);
    });
    if (threadIdx.x == 0) a.draw_cnt[(size_t)b * kCntStride] = 0u;
}

// ---------------------------------------------------------------------------
// Greedy prefix match: one thread per sequence.
// ---------------------------------------------------------------------------
__global__ void k_greedy_prefix(Shape sh, const int32_t* gidx, int32_t* out_tokens, int32_t* out_num) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= sh.B) return;
    const int K = sh.K;
    const int Kb = seq_len(sh, b);
    const int32_t* g = gidx + (size_t)b * (K + 1);
    const int32_t* d = sh.tokens + (size_t)b * K;
    int j = Kb;
    for (int k = 0; k < Kb; ++k)
        if (d[k] != g[k]) {
            j = k;
            break;
        }
    int32_t* out = out_tokens + (size_t)b * (K + 1);
    for (int k = 0; k < j; ++k) out[k] = d[k];
    out[j] = g[j];
    for (int k = j + 1; k <= K; ++k) out[k] = -1;
    out_num[b] = j;
    count_accepts(sh, b, j);
}

// Greedy verification in one launch (drafted sequences, fewer than
// kSplitRows of them).  Each workgroup takes one target row's lowest-index
// argmax, stores it with an agent-scope store, waits for the store and counts
// its row on the sequence's counter; the last of the sequence's live rows to
// arrive matches the prefix (the greedy rule of "DFlash", section 4: the
// longest run of drafted tokens equal to the target's argmax, then the
// target's token at the first mismatch, or the bonus token after the last
// draft) and writes the outputs.  When acceptance counts are asked for, the
// last sequence to finish counts the batch's totals per position and writes
// them (no clearing, no atomics on them).  The counters are zero between
// calls: each last arrival resets its own.
struct GreedyArgs {
    Shape sh;
    int32_t* gidx;        // [n_trows] row argmaxes
    int32_t* out_tokens;  // [B][K+1]
    int32_t* out_num;     // [B]
    unsigned* cnt;        // B sequence counters, then the batch counter, kCntStride apart
};

struct GreedyShared {
    int flag, j;
    int jb[kSplitRows];
};

// The row's part, for the whole workgroup: store the argmax am of row `row`
// (of sequence b), count it, and, in the last live row of the sequence to
// arrive, write the sequence's outputs (and, in the last sequence, the
// batch's acceptance counts).
__device__ __forceinline__ void greedy_arrive(const GreedyArgs& g, int row, int32_t am, GreedyShared& S) {
    const Shape& sh = g.sh;
    const int K = sh.K, b = row / (K + 1), Kb = seq_len(sh, b);
    const int nt = (int)blockDim.x;
    if (threadIdx.x == 0) {
        st_agent(&g.gidx[row], am);
        wait_stores();
        S.flag = __hip_atomic_fetch_add(&g.cnt[(size_t)b * kCntStride], 1u, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) == (unsigned)Kb;
        S.j = Kb;
    }
    __syncthreads();
    if (!S.flag) return;
    // the first position k < K_b whose drafted token differs from the argmax
    const int32_t* d = sh.tokens + (size_t)b * K;
    const int32_t* gi = g.gidx + (size_t)b * (K + 1);
    for (int k0 = 0; k0 < Kb; k0 += nt) {
        const int k = k0 + (int)threadIdx.x;
        if (k < Kb && d[k] != ld_agent(&gi[k])) atomicMin(&S.j, k);
        __syncthreads();
        if (S.j < Kb) break;
    }
    const int j = S.j;
    const int32_t gj = ld_agent(&gi[j]);
    int32_t* out = g.out_tokens + (size_t)b * (K + 1);
    for (int k = threadIdx.x; k <= K; k += nt) out[k] = k < j ? d[k] : (k == j ? gj : -1);
    const bool counts = sh.tested || sh.accepted;
    __syncthreads();  // every thread has read S.j
    if (threadIdx.x == 0) {
        g.cnt[(size_t)b * kCntStride] = 0u;
        if (counts) {
            st_agent(&g.out_num[b], j);
            wait_stores();
            S.flag = __hip_atomic_fetch_add(&g.cnt[(size_t)sh.B * kCntStride], 1u, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(sh.B - 1);
        } else {
            g.out_num[b] = j;
            S.flag = 0;
        }
    }
    __syncthreads();
    if (!S.flag) return;
    // the batch's last sequence: tests ran at positions k <= j_b, k < K_b,
    // and accepted at k < j_b
    for (int bb = threadIdx.x; bb < sh.B; bb += nt) S.jb[bb] = ld_agent(&g.out_num[bb]);
    __syncthreads();
    for (int k = threadIdx.x; k < K; k += nt) {
        int t = 0, ac = 0;
        for (int bb = 0; bb < sh.B; ++bb) {
            const int jb = S.jb[bb];
            t += k < min(jb + 1, seq_len(sh, bb)) ? 1 : 0;
            ac += k < jb ? 1 : 0;
        }
        if (sh.tested) sh.tested[k] = t;
        if (sh.accepted) sh.accepted[k] = ac;
    }
    if (threadIdx.x == 0) g.cnt[(size_t)sh.B * kCntStride] = 0u;
}

__global__ void __launch_bounds__(kRB) k_greedy_rows(GreedyArgs g) {
    __shared__ u64 s_red[kRW];
    __shared__ GreedyShared S;
    const Shape& sh = g.sh;
    const int row = blockIdx.x;
    if (!row_live(sh, row)) return;
    const int32_t am = sh.tdt == DT_BF16 ? argmax_body<DT_BF16>(sh, row, s_red) : argmax_body<DT_F32>(sh, row, s_red);
    greedy_arrive(g, row, am, S);
}

// Copy row records to the caller's stats arrays.
__global__ void k_copy_stats(const RowRec* rec, int n_trows, int n_drows, spec_row_stats_t* tstats,
                             spec_row_stats_t* dstats) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_trows) {
        if (tstats) tstats[i] = rec[i].s;
    } else if (i < n_trows + n_drows) {
        if (dstats) dstats[i - n_trows] = rec[i].s;
    }
}

// Diagnostic: uniforms of the accept tests and draws.
__global__ void k_uniforms(uint64_t seed, int B, int K, double* ua, double* us) {
    const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
    const long long na = (long long)B * K, ns = (long long)B * (K + 1);
    if (ua && i < na)
        ua[i] = uniform24(draw_block(seed, (uint32_t)(i / K), (uint32_t)(i % K), PURPOSE_ACCEPT));
    if (us && i < ns)
        us[i] = uniform53(draw_block(seed, (uint32_t)(i / (K + 1)), (uint32_t)(i % (K + 1)), PURPOSE_SAMPLE));
}

}  // namespace sv
