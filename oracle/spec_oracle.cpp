/*
 * spec_oracle.cpp — CPU reference for batched speculative-decoding
 * verification.  TEST INFRASTRUCTURE ONLY (see spec_oracle.h): plain,
 * single-threaded, fp64 throughout, written for a reader to check against
 * the pages by eye.  No blocking, fusion or reordering beyond what the
 * definitions state; library primitives (std::nth_element, std::sort, exp)
 * serve as steps.
 */
#include "spec_oracle.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <functional>
#include <limits>
#include <vector>

namespace {

const double kInf = std::numeric_limits<double>::infinity();
const double kNaN = std::numeric_limits<double>::quiet_NaN();

/* Widen one stored logit to double (exact for both formats). */
double load_logit(const void* row, int dtype, long long i) {
    if (dtype == ORACLE_F32) {
        float f;
        std::memcpy(&f, static_cast<const char*>(row) + 4 * i, 4);
        return f;
    }
    uint16_t h;
    std::memcpy(&h, static_cast<const char*>(row) + 2 * i, 2);
    uint32_t bits = static_cast<uint32_t>(h) << 16; /* bf16 is the high half */
    float f;
    std::memcpy(&f, &bits, 4);
    return f;
}

size_t dtype_size(int dtype) { return dtype == ORACLE_F32 ? 4 : 2; }

bool dtype_ok(int dtype) { return dtype == ORACLE_F32 || dtype == ORACLE_BF16; }

/* The processed distribution of one row plus its diagnostics. */
struct Row {
    std::vector<double> prob; /* length V */
    oracle_row_info info;
};

/*
 * Logit processing, in the order temperature -> top-k -> softmax -> top-p
 * on the renormalised top-k set -> renormalise (the threatfrontier page,
 * "Why the output is identical", asks only that top-k and top-p be applied
 * the same way to target and draft; this order is the reading taken).
 *   1. s_i = x_i / T (FlashMap page, section 5: logits / temperature before
 *      the softmax).
 *   2. top-k: tau = k-th largest s; keep s_i >= tau, so ties at tau are kept
 *      and more than k tokens may survive.  top_k <= 0 or >= V: off.
 *   3. m = max kept s, w_i = exp(s_i - m) on kept tokens, Z = sum w.
 *   4. top-p (top_p < 1): visit groups of equal s in descending order; a
 *      group is kept while the mass of all strictly greater groups, divided
 *      by Z, is below top_p.  The top group is always kept, the group that
 *      crosses top_p is kept whole.
 *   5. prob_i = w_i / (sum of w over kept tokens).
 */
int process_row(const void* row, int dtype, int V, double T, int top_k,
                double top_p, Row& out) {
    std::vector<double> s(V);
    std::vector<double> x(V);
    for (int i = 0; i < V; ++i) {
        x[i] = load_logit(row, dtype, i);
        s[i] = x[i] / T;
    }

    std::vector<char> kept(V, 1);
    if (top_k > 0 && top_k < V) {
        std::vector<double> tmp(s);
        std::nth_element(tmp.begin(), tmp.begin() + (top_k - 1), tmp.end(),
                         std::greater<double>());
        const double tau = tmp[top_k - 1];
        for (int i = 0; i < V; ++i) kept[i] = s[i] >= tau;
    }

    double m = -kInf;
    for (int i = 0; i < V; ++i)
        if (kept[i] && s[i] > m) m = s[i];
    if (!(m > -kInf)) return 1; /* every kept logit is -inf: unsupported */

    std::vector<double> w(V, 0.0);
    for (int i = 0; i < V; ++i)
        if (kept[i]) w[i] = std::exp(s[i] - m);
    double Z = 0.0;
    for (int i = 0; i < V; ++i) Z += w[i];

    double margin = kInf;
    if (top_p < 1.0) {
        std::vector<int> order;
        for (int i = 0; i < V; ++i)
            if (kept[i]) order.push_back(i);
        std::sort(order.begin(), order.end(), [&](int a, int b) {
            if (s[a] != s[b]) return s[a] > s[b];
            return a < b;
        });
        double excl = 0.0; /* mass of all strictly greater groups */
        bool cut = false;
        size_t g = 0;
        while (g < order.size()) {
            size_t h = g;
            double group_mass = 0.0;
            while (h < order.size() && s[order[h]] == s[order[g]]) {
                group_mass += w[order[h]];
                ++h;
            }
            if (!cut) {
                const double frac = excl / Z;
                if (frac < top_p) {
                    margin = std::min(margin, top_p - frac);
                } else {
                    margin = std::min(margin, frac - top_p);
                    cut = true;
                }
            }
            if (cut)
                for (size_t t = g; t < h; ++t) {
                    kept[order[t]] = 0;
                    w[order[t]] = 0.0;
                }
            excl += group_mass;
            g = h;
        }
    }

    double Zk = 0.0;
    for (int i = 0; i < V; ++i) Zk += w[i];

    out.prob.assign(V, 0.0);
    double thresh = kInf;
    int n_kept = 0;
    for (int i = 0; i < V; ++i) {
        out.prob[i] = w[i] / Zk;
        if (kept[i]) {
            ++n_kept;
            if (x[i] < thresh) thresh = x[i];
        }
    }
    out.info.max_scaled = m;
    out.info.z_kept = Zk;
    out.info.thresh = thresh;
    out.info.n_kept = n_kept;
    out.info.reserved = 0;
    out.info.nucleus_margin = margin;
    out.info.prob_at_token = kNaN;
    return 0;
}

void philox_block(uint64_t seed, uint32_t b, uint32_t k, uint32_t purpose,
                  uint32_t out[4]) {
    const uint32_t counter[4] = {b, k, purpose, 0u};
    const uint32_t key[2] = {static_cast<uint32_t>(seed),
                             static_cast<uint32_t>(seed >> 32)};
    oracle_philox4x32_10(counter, key, out);
}

}  // namespace

extern "C" {

/*
 * Philox4x32-10 (SC'11 paper cited in the header).  Each round multiplies
 * counter words 0 and 2 by the two round multipliers, takes the 64-bit
 * products apart into high and low halves, and mixes the high halves with
 * the other two counter words and the key; the key is advanced by the two
 * Weyl increments between rounds (ten rounds, nine key advances).
 */
void oracle_philox4x32_10(const uint32_t counter[4], const uint32_t key[2],
                          uint32_t out[4]) {
    uint32_t c0 = counter[0], c1 = counter[1], c2 = counter[2], c3 = counter[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        if (round > 0) {
            k0 += 0x9E3779B9u;
            k1 += 0xBB67AE85u;
        }
        const uint64_t prod0 = static_cast<uint64_t>(0xD2511F53u) * c0;
        const uint64_t prod1 = static_cast<uint64_t>(0xCD9E8D57u) * c2;
        const uint32_t n0 = static_cast<uint32_t>(prod1 >> 32) ^ c1 ^ k0;
        const uint32_t n1 = static_cast<uint32_t>(prod1);
        const uint32_t n2 = static_cast<uint32_t>(prod0 >> 32) ^ c3 ^ k1;
        const uint32_t n3 = static_cast<uint32_t>(prod0);
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

double oracle_u24(uint64_t seed, uint32_t b, uint32_t k, uint32_t purpose) {
    uint32_t w[4];
    philox_block(seed, b, k, purpose, w);
    return static_cast<double>(w[0] >> 8) * 0x1p-24;
}

/* 53-bit uniform from two words (Matsumoto & Nishimura's genrand_res53
 * construction: 27 high bits of one word, 26 of the next). */
double oracle_u53(uint64_t seed, uint32_t b, uint32_t k, uint32_t purpose) {
    uint32_t w[4];
    philox_block(seed, b, k, purpose, w);
    const double hi = static_cast<double>(w[0] >> 5);
    const double lo = static_cast<double>(w[1] >> 6);
    return (hi * 67108864.0 + lo) * 0x1p-53;
}

int oracle_process_row(const void* row, int dtype, int V, double temperature,
                       int top_k, double top_p, double* prob,
                       oracle_row_info* info) {
    if (!row || V < 1 || !dtype_ok(dtype)) return 1;
    if (!(temperature > 0.0) || !std::isfinite(temperature)) return 1;
    if (!(top_p > 0.0 && top_p <= 1.0)) return 1;
    Row r;
    if (process_row(row, dtype, V, temperature, top_k, top_p, r)) return 1;
    if (prob) std::memcpy(prob, r.prob.data(), sizeof(double) * V);
    if (info) *info = r.info;
    return 0;
}

int oracle_verify_greedy(const void* target, int target_dtype,
                         const int32_t* draft_tokens, int B, int K, int V,
                         int32_t* out_tokens, int32_t* out_num_accepted) {
    if (B < 0 || K < 0 || V < 1 || !dtype_ok(target_dtype)) return 1;
    if (B == 0) return 0;
    if (!target || !out_tokens || !out_num_accepted || (K > 0 && !draft_tokens))
        return 1;
    const size_t esz = dtype_size(target_dtype);
    for (int b = 0; b < B; ++b) {
        /* g_k = argmax of target row k, lowest index among equal maxima. */
        std::vector<int> g(K + 1);
        for (int k = 0; k <= K; ++k) {
            const void* row = static_cast<const char*>(target) +
                              (static_cast<size_t>(b) * (K + 1) + k) * V * esz;
            int best = 0;
            double best_v = load_logit(row, target_dtype, 0);
            for (int i = 1; i < V; ++i) {
                const double v = load_logit(row, target_dtype, i);
                if (v > best_v) {
                    best_v = v;
                    best = i;
                }
            }
            g[k] = best;
        }
        /* Accept the longest prefix where the draft equals the target's
         * argmax; at the first mismatch the output is the target argmax of
         * that row (row K's argmax, the bonus, when all K match). */
        int j = K;
        for (int k = 0; k < K; ++k)
            if (draft_tokens[static_cast<size_t>(b) * K + k] != g[k]) {
                j = k;
                break;
            }
        int32_t* out = out_tokens + static_cast<size_t>(b) * (K + 1);
        for (int k = 0; k < j; ++k) out[k] = draft_tokens[static_cast<size_t>(b) * K + k];
        out[j] = g[j];
        for (int k = j + 1; k <= K; ++k) out[k] = -1;
        out_num_accepted[b] = j;
    }
    return 0;
}

int oracle_verify(const void* target, int target_dtype, const void* draft,
                  int draft_dtype, const int32_t* draft_tokens, int B, int K,
                  int V, double temperature, int top_k, double top_p,
                  uint64_t seed, int seq_base, int32_t* out_tokens,
                  int32_t* out_num_accepted, double* accept_margin,
                  double* sample_margin, oracle_row_info* target_info,
                  oracle_row_info* draft_info) {
    if (B < 0 || K < 0 || V < 1 || seq_base < 0) return 1;
    if (!dtype_ok(target_dtype)) return 1;
    if (!(temperature >= 0.0) || !std::isfinite(temperature)) return 1;
    if (!(top_p > 0.0 && top_p <= 1.0)) return 1;
    if (temperature == 0.0)
        return oracle_verify_greedy(target, target_dtype, draft_tokens, B, K, V,
                                    out_tokens, out_num_accepted);
    if (B == 0) return 0;
    if (!target || !out_tokens || !out_num_accepted) return 1;
    if (K > 0 && (!draft || !draft_tokens || !dtype_ok(draft_dtype))) return 1;

    const size_t tsz = dtype_size(target_dtype);
    const size_t dsz = K > 0 ? dtype_size(draft_dtype) : 0;

    for (int b = 0; b < B; ++b) {
        const uint32_t gb = static_cast<uint32_t>(seq_base + b);

        /* Process every row of this sequence: p_0..p_K and q_0..q_{K-1}. */
        std::vector<Row> P(K + 1), Q(K);
        for (int k = 0; k <= K; ++k) {
            const void* row = static_cast<const char*>(target) +
                              (static_cast<size_t>(b) * (K + 1) + k) * V * tsz;
            if (process_row(row, target_dtype, V, temperature, top_k, top_p, P[k]))
                return 2;
        }
        for (int k = 0; k < K; ++k) {
            const void* row = static_cast<const char*>(draft) +
                              (static_cast<size_t>(b) * K + k) * V * dsz;
            if (process_row(row, draft_dtype, V, temperature, top_k, top_p, Q[k]))
                return 2;
        }

        /* Probability of each drafted token under p_k and q_k; a token
         * outside [0, V) has p = q = 0 and is therefore rejected. */
        std::vector<double> pd(K, 0.0), qd(K, 0.0);
        for (int k = 0; k < K; ++k) {
            const int x = draft_tokens[static_cast<size_t>(b) * K + k];
            if (x >= 0 && x < V) {
                pd[k] = P[k].prob[x];
                qd[k] = Q[k].prob[x];
                P[k].info.prob_at_token = pd[k];
                Q[k].info.prob_at_token = qd[k];
            }
        }

        /*
         * Accept test, left to right (FlashMap page section 4; DFlash page
         * section 4; threatfrontier "Why the output is identical"): draw
         * u ~ U[0,1) and accept d_k when u * q < p, i.e. with probability
         * min(1, p/q).  Strict '<' with u in [0,1) is the reading taken:
         * p = 0 is never accepted and p >= q is always accepted.  When
         * q = 0 the same product form accepts exactly when p > 0.
         * The first rejection ends the scan (everything after it is
         * discarded).
         */
        int j = K;
        for (int k = 0; k < K; ++k) {
            const double u = oracle_u24(seed, gb, static_cast<uint32_t>(k),
                                        ORACLE_PURPOSE_ACCEPT);
            const double p = pd[k], q = qd[k];
            if (accept_margin)
                accept_margin[static_cast<size_t>(b) * K + k] =
                    q > 0.0 ? std::fabs(u * q - p) / q : kInf;
            if (!(u * q < p)) {
                j = k;
                break;
            }
        }
        if (accept_margin)
            for (int k = j + 1; k < K; ++k)
                accept_margin[static_cast<size_t>(b) * K + k] = kNaN;

        /*
         * Stop token.  After a rejection at position j < K: sample from the
         * normalised residual max(0, p_j - q_j) (FlashMap page section 4,
         * recovery distribution).  If rounding leaves no residual mass
         * (S = 0; impossible in exact arithmetic after a rejection), sample
         * from p_j instead.  When all K drafts are accepted: sample the bonus
         * token from p_K (DFlash page section 4: the target gives K+1
         * distributions).  Inverse CDF in ascending token order with a
         * 53-bit uniform: the first y whose running sum exceeds t = u * S.
         */
        std::vector<double> r(V);
        double S = 0.0;
        if (j < K) {
            for (int i = 0; i < V; ++i) {
                const double d = P[j].prob[i] - Q[j].prob[i];
                r[i] = d > 0.0 ? d : 0.0;
            }
            for (int i = 0; i < V; ++i) S += r[i];
        }
        if (j == K || S == 0.0) {
            for (int i = 0; i < V; ++i) r[i] = P[j].prob[i];
            S = 0.0;
            for (int i = 0; i < V; ++i) S += r[i];
        }
        const double t = oracle_u53(seed, gb, static_cast<uint32_t>(j),
                                    ORACLE_PURPOSE_SAMPLE) * S;
        int y = -1, last_pos = -1;
        double cum = 0.0, margin = 0.0;
        for (int i = 0; i < V; ++i) {
            if (!(r[i] > 0.0)) continue;
            last_pos = i;
            const double prev = cum;
            cum += r[i];
            if (y < 0 && cum > t) {
                y = i;
                margin = std::min(t - prev, cum - t) / S;
            }
        }
        if (y < 0) { /* rounding left t at or past the total */
            y = last_pos;
            margin = 0.0;
        }
        if (sample_margin) sample_margin[b] = margin;

        int32_t* out = out_tokens + static_cast<size_t>(b) * (K + 1);
        for (int k = 0; k < j; ++k) out[k] = draft_tokens[static_cast<size_t>(b) * K + k];
        out[j] = y;
        for (int k = j + 1; k <= K; ++k) out[k] = -1;
        out_num_accepted[b] = j;

        if (target_info)
            for (int k = 0; k <= K; ++k)
                target_info[static_cast<size_t>(b) * (K + 1) + k] = P[k].info;
        if (draft_info)
            for (int k = 0; k < K; ++k)
                draft_info[static_cast<size_t>(b) * K + k] = Q[k].info;
    }
    return 0;
}

/*
 * Point-mass drafts.  A drafter that proposes d_k with certainty has
 * q_k = delta(d_k); top-k and top-p leave a point mass unchanged.  The
 * rejection test ("Why the output is identical" on the same page; FlashMap
 * page section 4) with q_k(d_k) = 1 accepts d_k with probability
 * min(1, p_k(d_k)), i.e. when u * 1 < p_k(d_k).  After the first rejection
 * at j < K the stop token comes from max(0, p_j - delta(d_j)) normalised:
 * p_j with d_j taken out.  After K acceptances the bonus token comes from
 * p_K.  Uniforms, inverse CDF and the S = 0 reading are those of
 * oracle_verify.
 */
int oracle_verify_point(const void* target, int target_dtype,
                        const int32_t* draft_tokens, int B, int K, int V,
                        double temperature, int top_k, double top_p,
                        uint64_t seed, int seq_base, int32_t* out_tokens,
                        int32_t* out_num_accepted, double* accept_margin,
                        double* sample_margin, oracle_row_info* target_info) {
    if (B < 0 || K < 0 || V < 1 || seq_base < 0) return 1;
    if (!dtype_ok(target_dtype)) return 1;
    if (!(temperature >= 0.0) || !std::isfinite(temperature)) return 1;
    if (!(top_p > 0.0 && top_p <= 1.0)) return 1;
    if (temperature == 0.0)
        return oracle_verify_greedy(target, target_dtype, draft_tokens, B, K, V,
                                    out_tokens, out_num_accepted);
    if (B == 0) return 0;
    if (!target || !out_tokens || !out_num_accepted) return 1;
    if (K > 0 && !draft_tokens) return 1;
    const size_t tsz = dtype_size(target_dtype);

    for (int b = 0; b < B; ++b) {
        const uint32_t gb = static_cast<uint32_t>(seq_base + b);
        const int32_t* d = draft_tokens + static_cast<size_t>(b) * K;

        std::vector<Row> P(K + 1);
        for (int k = 0; k <= K; ++k) {
            const void* row = static_cast<const char*>(target) +
                              (static_cast<size_t>(b) * (K + 1) + k) * V * tsz;
            if (process_row(row, target_dtype, V, temperature, top_k, top_p, P[k]))
                return 2;
        }

        /* q_k(x) is 1 at x = d_k and 0 elsewhere; a token outside [0, V)
         * has p = 0 and is rejected. */
        auto q_of = [&](int k, int x) { return x == d[k] ? 1.0 : 0.0; };

        int j = K;
        for (int k = 0; k < K; ++k) {
            const int x = d[k];
            const double p = (x >= 0 && x < V) ? P[k].prob[x] : 0.0;
            if (x >= 0 && x < V) P[k].info.prob_at_token = p;
            const double q = 1.0;
            const double u = oracle_u24(seed, gb, static_cast<uint32_t>(k),
                                        ORACLE_PURPOSE_ACCEPT);
            if (accept_margin)
                accept_margin[static_cast<size_t>(b) * K + k] = std::fabs(u * q - p) / q;
            if (!(u * q < p)) {
                j = k;
                break;
            }
        }
        if (accept_margin)
            for (int k = j + 1; k < K; ++k)
                accept_margin[static_cast<size_t>(b) * K + k] = kNaN;

        std::vector<double> r(V);
        double S = 0.0;
        if (j < K) {
            for (int i = 0; i < V; ++i) {
                const double diff = P[j].prob[i] - q_of(j, i);
                r[i] = diff > 0.0 ? diff : 0.0;
            }
            for (int i = 0; i < V; ++i) S += r[i];
        }
        if (j == K || S == 0.0) {
            for (int i = 0; i < V; ++i) r[i] = P[j].prob[i];
            S = 0.0;
            for (int i = 0; i < V; ++i) S += r[i];
        }
        const double t = oracle_u53(seed, gb, static_cast<uint32_t>(j),
                                    ORACLE_PURPOSE_SAMPLE) * S;
        int y = -1, last_pos = -1;
        double cum = 0.0, margin = 0.0;
        for (int i = 0; i < V; ++i) {
            if (!(r[i] > 0.0)) continue;
            last_pos = i;
            const double prev = cum;
            cum += r[i];
            if (y < 0 && cum > t) {
                y = i;
                margin = std::min(t - prev, cum - t) / S;
            }
        }
        if (y < 0) {
            y = last_pos;
            margin = 0.0;
        }
        if (sample_margin) sample_margin[b] = margin;

        int32_t* out = out_tokens + static_cast<size_t>(b) * (K + 1);
        for (int k = 0; k < j; ++k) out[k] = d[k];
        out[j] = y;
        for (int k = j + 1; k <= K; ++k) out[k] = -1;
        out_num_accepted[b] = j;

        if (target_info)
            for (int k = 0; k <= K; ++k)
                target_info[static_cast<size_t>(b) * (K + 1) + k] = P[k].info;
    }
    return 0;
}

int oracle_verify_tree(const void* target, int target_dtype,
                       const int32_t* node_tokens, const int32_t* parents, int B,
                       int N, int V, double temperature, int top_k, double top_p,
                       uint64_t seed, int seq_base, int32_t* out_tokens,
                       int32_t* out_num_accepted, int32_t* out_path,
                       double* accept_margin, double* sample_margin,
                       oracle_row_info* target_info) {
    if (B < 0 || N < 0 || V < 1 || seq_base < 0) return 1;
    if (!dtype_ok(target_dtype)) return 1;
    if (!(temperature >= 0.0) || !std::isfinite(temperature)) return 1;
    if (!(top_p > 0.0 && top_p <= 1.0)) return 1;
    if (B == 0) return 0;
    if (!target || !out_tokens || !out_num_accepted) return 1;
    if (N > 0 && (!node_tokens || !parents)) return 1;
    const size_t tsz = dtype_size(target_dtype);
    const bool greedy = temperature == 0.0;

    for (int b = 0; b < B; ++b) {
        const uint32_t gb = static_cast<uint32_t>(seq_base + b);
        const int32_t* tok = node_tokens + static_cast<size_t>(b) * N;
        const int32_t* par = parents + static_cast<size_t>(b) * N;
        auto row_of = [&](int r) {
            return static_cast<const char*>(target) +
                   (static_cast<size_t>(b) * (N + 1) + r) * V * tsz;
        };
        /* children of node u (u = -1: the root) in index order; a node is
         * a child of its parent only if the parent index is below its own */
        auto children = [&](int u) {
            std::vector<int> c;
            for (int i = u + 1; i < N; ++i)
                if (par[i] == u) c.push_back(i);
            return c;
        };
        if (accept_margin)
            for (int i = 0; i < N; ++i) accept_margin[static_cast<size_t>(b) * N + i] = kNaN;

        std::vector<int> path;
        int u = -1;  // current node
        int y = -1;  // the last token
        double margin = 0.0;
        if (greedy) {
            for (;;) {
                /* argmax of the current row, lowest index among equal maxima */
                const char* row = row_of(u + 1);
                int g = 0;
                double gv = load_logit(row, target_dtype, 0);
                for (int i = 1; i < V; ++i) {
                    const double v = load_logit(row, target_dtype, i);
                    if (v > gv) {
                        gv = v;
                        g = i;
                    }
                }
                int next = -1;
                for (int c : children(u))
                    if (tok[c] == g) {
                        next = c;
                        break;
                    }
                if (next < 0) {
                    y = g;
                    break;
                }
                path.push_back(next);
                u = next;
            }
        } else {
            std::vector<Row> P(N + 1);
            for (int r = 0; r <= N; ++r)
                if (process_row(row_of(r), target_dtype, V, temperature, top_k, top_p, P[r]))
                    return 2;
            std::vector<double> p;
            for (;;) {
                const int r = u + 1;
                p = P[r].prob;
                int next = -1;
                for (int c : children(u)) {
                    const int x = tok[c];
                    const double px = (x >= 0 && x < V) ? p[x] : 0.0;
                    const double uc = oracle_u24(seed, gb, static_cast<uint32_t>(c),
                                                 ORACLE_PURPOSE_ACCEPT);
                    if (accept_margin)
                        accept_margin[static_cast<size_t>(b) * N + c] = std::fabs(uc - px);
                    if (uc < px) {
                        next = c;
                        break;
                    }
                    /* rejected: remove x and renormalise what is left */
                    if (x >= 0 && x < V && p[x] > 0.0) {
                        p[x] = 0.0;
                        double s = 0.0;
                        for (int i = 0; i < V; ++i) s += p[i];
                        if (s > 0.0)
                            for (int i = 0; i < V; ++i) p[i] /= s;
                    }
                }
                if (next < 0) break;
                path.push_back(next);
                u = next;
            }
            /* the draw: from what is left of p, or the row itself when no
             * mass is left (a leaf has p equal to its row) */
            const int r = u + 1;
            double S = 0.0;
            for (int i = 0; i < V; ++i) S += p[i];
            if (!(S > 0.0)) {
                p = P[r].prob;
                S = 0.0;
                for (int i = 0; i < V; ++i) S += p[i];
            }
            const double t = oracle_u53(seed, gb, static_cast<uint32_t>(r),
                                        ORACLE_PURPOSE_SAMPLE) * S;
            int last_pos = -1;
            double cum = 0.0;
            for (int i = 0; i < V; ++i) {
                if (!(p[i] > 0.0)) continue;
                last_pos = i;
                const double prev = cum;
                cum += p[i];
                if (y < 0 && cum > t) {
                    y = i;
                    margin = std::min(t - prev, cum - t) / S;
                }
            }
            if (y < 0) {
                y = last_pos;
                margin = 0.0;
            }
            if (target_info)
                for (int k = 0; k <= N; ++k)
                    target_info[static_cast<size_t>(b) * (N + 1) + k] = P[k].info;
        }
        if (sample_margin) sample_margin[b] = margin;

        const int n = static_cast<int>(path.size());
        int32_t* out = out_tokens + static_cast<size_t>(b) * (N + 1);
        for (int k = 0; k < n; ++k) out[k] = tok[path[k]];
        out[n] = y;
        for (int k = n + 1; k <= N; ++k) out[k] = -1;
        out_num_accepted[b] = n;
        if (out_path) {
            int32_t* op = out_path + static_cast<size_t>(b) * N;
            for (int k = 0; k < N; ++k) op[k] = k < n ? path[k] : -1;
        }
    }
    return 0;
}

}  // extern "C"
