// seq_kernels.h — per-sequence kernels: the accept scan over K drafted
// positions and the draw of the stop token.
//
//  k_seq_filtered : filtered rows (top-k / top-p).  p_j is nonzero only on the
//                   stop target row's kept set, stored sorted by index by
//                   k_row, so the residual max(0, p_j - q_j) is evaluated on
//                   that list (with the draft logits stored beside it).  One
//                   workgroup per (sequence, possible stop position).
//  k_draw_sums / k_draw_pick : unfiltered rows.  The residual is spread over
//                   the whole vocabulary: chunk sums over the stop row pair in
//                   fp64, then one workgroup per sequence locates the draw.
//  k_greedy_prefix : greedy prefix match from the per-row argmax.
//
// k_draw_sums / k_draw_pick also serve token trees (filtered or not): there a
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

struct SeqArgs {
    Shape sh;
    double inv_T;
    uint64_t seed;
    const RowRec* rec;
    const uint2* kept;
    const int* kept_n;
    const float* kept_d;  // draft logit of each listed token (stop positions j < K)
    const double* kept_p; // p of each listed token
    double2* chunk_sum;   // [B][n_chunks] (.x residual, .y p)
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
template <bool kTree>
__device__ __forceinline__ bool stop_is_bonus(const SeqArgs& a, int b, int j) {
    if constexpr (kTree) return a.tstop[b].n_ex == 0;
    else return j >= seq_len(a.sh, b);
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
// Unfiltered: chunk sums, then the pick.
// ---------------------------------------------------------------------------
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

// p_j and the residual max(0, p_j - q_j) of the kCPT tokens from lo on, in
// fp64 (the same arithmetic wherever a chunk is summed or searched).
template <int TDT, int DDT>
__device__ __forceinline__ void run_terms(const StopRow& s, double inv_T, int lo, int V, double (&p)[kCPT],
                                          double (&r)[kCPT]) {
    float xt[kCPT], xd[kCPT];
    load_run<TDT>(s.tp, lo, V, xt);
    // without a draft row the target row is read again and ignored
    load_run<DDT>(s.has_draft ? s.dp : s.tp, lo, V, xd);
    const double inv_zt = 1.0 / s.zt, inv_zd = 1.0 / s.zd;
    // removed tokens of a tree's stop row inside [lo, lo + kCPT)
    uint32_t exm = 0u;
    for (int e = 0; e < s.n_ex; ++e) {
        const uint32_t d = (uint32_t)(s.ex[e] - lo);
        if (d < (uint32_t)kCPT) exm |= 1u << d;
    }
#pragma unroll
    for (int e = 0; e < kCPT; ++e) {
        p[e] = xt[e] >= s.thr_t ? exp(((double)xt[e] - (double)s.Mt) * inv_T) * inv_zt : 0.0;
        const double q = (s.has_draft && xd[e] >= s.thr_d) ? exp(((double)xd[e] - (double)s.Md) * inv_T) * inv_zd
                                                           : ((lo + e == s.dtok || ((exm >> e) & 1u)) ? 1.0 : 0.0);
        const double d = p[e] - q;
        r[e] = d > 0.0 ? d : 0.0;
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

// Chunk sums of the stop row pair: one workgroup per (sequence, chunk).
// (Four chunks per workgroup, one round of workgroups for large batches, was
// slower: each workgroup's chain of loads, scans and barriers grew.)
template <bool kTree>
__global__ void __launch_bounds__(kSB) k_draw_sums(SeqArgs a) {
    __shared__ double s_wa[kSB / 64], s_wb[kSB / 64];
    __shared__ int s_j;
    const int b = blockIdx.x / a.n_chunks;
    const int c = blockIdx.x % a.n_chunks;
    if (threadIdx.x < 64) {
        const int j = stop_of<kTree>(a, b);
        if (threadIdx.x == 0) s_j = j;
    }
    __syncthreads();
    const StopRow s = stop_row<kTree>(a, b, s_j);
    with_dtypes(s, [&](auto tt, auto dt) {
        double p[kCPT], r[kCPT];
        run_terms<decltype(tt)::value, decltype(dt)::value>(s, a.inv_T, c * kChunk + threadIdx.x * kCPT, a.sh.V, p,
                                                             r);
        double sr = 0.0, sp = 0.0;
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
            sr += r[e];
            sp += p[e];
        }
        double er, ep, tr, tp;
        seq_excl_scan2(sr, sp, s_wa, s_wb, er, ep, tr, tp);
        if (threadIdx.x == 0) a.chunk_sum[(size_t)b * a.n_chunks + c] = make_double2(tr, tp);
    });
}

// One workgroup per sequence: the chunk holding the draw point (chunk sums
// in chunk order, thread t holding chunks t, t + kSB, ...), then the token
// inside it from the same per-thread terms.
template <bool kTree>
__global__ void __launch_bounds__(kSB) k_draw_pick(SeqArgs a) {
    __shared__ double s_wa[kSB / 64], s_wb[kSB / 64], s_run;
    __shared__ int s_j, s_cstar;
    __shared__ int s_last[kSB / 64], s_first[kSB / 64];
    const int b = blockIdx.x;
    const int K = a.sh.K, V = a.sh.V;
    if (threadIdx.x < 64) {
        const int j = stop_of<kTree>(a, b);
        if (threadIdx.x == 0) {
            s_j = j;
            s_cstar = 0;  // stays if no chunk holds mass
            s_run = 0.0;
        }
    }
    const double2* cs = a.chunk_sum + (size_t)b * a.n_chunks;
    // this thread's chunks are contiguous: [c0, c1)
    const int per = (a.n_chunks + kSB - 1) / kSB;
    const int c0 = min((int)threadIdx.x * per, a.n_chunks), c1 = min(c0 + per, a.n_chunks);
    double mr = 0.0, mp = 0.0;
    for (int cc = c0; cc < c1; ++cc) {
        const double2 v = cs[cc];
        mr += v.x;
        mp += v.y;
    }
    double er, ep, tr, tp;
    seq_excl_scan2(mr, mp, s_wa, s_wb, er, ep, tr, tp);  // (its barrier also publishes s_j)
    const int j = s_j;
    const bool usep = stop_is_bonus<kTree>(a, b, j) || !(tr > 0.0);
    const double S = usep ? tp : tr;
    const double t = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)j, PURPOSE_SAMPLE)) * S;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    // the thread whose chunk range holds t (the last with mass starting at or
    // before t; else the first with mass), then the chunk inside its range
    auto locate = [&](double mine, double ex) {
        const unsigned long long mc = __ballot(mine > 0.0 && ex <= t);
        const unsigned long long mf = __ballot(mine > 0.0);
        __syncthreads();
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
        return tau >= 0 ? tau : first;
    };
    const int tc = locate(usep ? mp : mr, usep ? ep : er);
    if ((int)threadIdx.x == tc) {
        double run = usep ? ep : er;
        int cstar = -1, last_nz = c0;
        double run_last = run;
        for (int cc = c0; cc < c1; ++cc) {
            const double sc = usep ? cs[cc].y : cs[cc].x;
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
        s_cstar = cstar;
        s_run = run;
    }
    __syncthreads();
    const int cstar = s_cstar;
    const double run = s_run;
    const StopRow s = stop_row<kTree>(a, b, j);
    const int lo = cstar * kChunk + threadIdx.x * kCPT;
    with_dtypes(s, [&](auto tt, auto dt) {
        double p[kCPT], r[kCPT];
        run_terms<decltype(tt)::value, decltype(dt)::value>(s, a.inv_T, lo, V, p, r);
        double sr = 0.0, sp = 0.0;
#pragma unroll
        for (int e = 0; e < kCPT; ++e) {
            sr += r[e];
            sp += p[e];
        }
        double er2, ep2, tr2, tp2;
        seq_excl_scan2(sr, sp, s_wa, s_wb, er2, ep2, tr2, tp2);
        const double mine = usep ? sp : sr;
        const double ex = run + (usep ? ep2 : er2);
        const int tau = locate(mine, ex);
        if ((int)threadIdx.x == tau) {
            double acc = ex;
            int y = -1, last = -1;
#pragma unroll
            for (int e = 0; e < kCPT; ++e) {
                const double w = usep ? p[e] : r[e];
                if (y < 0 && w > 0.0) {
                    last = lo + e;
                    acc += w;
                    if (acc > t) y = lo + e;
                }
            }
            write_outputs<kTree>(a, b, j, y >= 0 ? y : last);
        }
    });
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
