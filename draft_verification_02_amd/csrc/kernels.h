// kernels.h — HIP kernels of the verifier (gfx950, wave64).
//
// Row numbering used by every kernel: rows [0, B*(K+1)) are target rows
// (b*(K+1) + k), rows [B*(K+1), B*(K+1) + B*K) are draft rows (b*K + k).
#pragma once

#include "device_common.h"
#include "../../include/spec_verify.h"

namespace sv {

// Per-row record kept in the workspace (public spec_row_stats_t + extras).
struct RowRec {
    spec_row_stats_t s;
    double z_all;  // sum over all tokens of exp((x - M)/T) (before filters)
    double pad;
};
static_assert(sizeof(spec_row_stats_t) == 32, "row stats layout");

struct Shape {
    const char* target;
    const char* draft;
    const int32_t* tokens;
    int B, K, V;
    int tdt, ddt;     // storage formats
    int tsz, dsz;     // bytes per element
    int n_trows, n_drows;
    int nt;           // streaming tiles per row
};

__device__ __forceinline__ const char* row_ptr(const Shape& sh, int row) {
    if (row < sh.n_trows) return sh.target + (size_t)row * sh.V * sh.tsz;
    return sh.draft + (size_t)(row - sh.n_trows) * sh.V * sh.dsz;
}
__device__ __forceinline__ int row_dt(const Shape& sh, int row) {
    return row < sh.n_trows ? sh.tdt : sh.ddt;
}
// Drafted token checked under this row, or -1 for a bonus row.
__device__ __forceinline__ int row_token(const Shape& sh, int row) {
    if (row < sh.n_trows) {
        const int b = row / (sh.K + 1), k = row % (sh.K + 1);
        return k < sh.K ? sh.tokens[(size_t)b * sh.K + k] : -1;
    }
    return sh.tokens[row - sh.n_trows];
}
__device__ __forceinline__ bool row_has_token(const Shape& sh, int row) {
    return row >= sh.n_trows || (row % (sh.K + 1)) < sh.K;
}

// ---------------------------------------------------------------------------
// Tile loader: kEPT logits per thread from elements [i0, i0 + n) of a row.
// Element order within a thread is increasing.  Missing elements are -inf and
// flagged invalid through `n`.  Fast path: 16-byte loads, each wave covering
// a contiguous 1 KiB span per load.
//   bf16: 4 loads x 8 elements, group g = j*256 + tid -> elements 8g..8g+7
//   f32 : 8 loads x 4 elements, group g = j*256 + tid -> elements 4g..4g+3
// index of v[slot]: see tile_index().
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ int tile_index(int slot) {
    constexpr int per = DT == DT_BF16 ? 8 : 4;
    const int j = slot / per, e = slot % per;
    return (j * kBlock + (int)threadIdx.x) * per + e;
}

template <int DT>
__device__ __forceinline__ void load_tile(const char* rowp, int i0, int n, float (&v)[kEPT]) {
    constexpr int esz = DT == DT_BF16 ? 2 : 4;
    constexpr int per = 16 / esz;
    constexpr int nload = kEPT / per;
    const char* base = rowp + (size_t)i0 * esz;
    const int tid = threadIdx.x;
    if ((((uintptr_t)base) & 15) == 0) {
        const int ngroups = n / per;
        u32x4 raw[nload];
#pragma unroll
        for (int j = 0; j < nload; ++j) {
            const int g = j * kBlock + tid;
            if (g < ngroups)
                raw[j] = ld16_nt(base + (size_t)g * 16);
            else
                raw[j] = u32x4{0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u, 0xFF80FF80u};
        }
#pragma unroll
        for (int j = 0; j < nload; ++j) {
            const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
            if (DT == DT_BF16) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    v[j * 8 + 2 * q] = bf16_lo(w[q]);
                    v[j * 8 + 2 * q + 1] = bf16_hi(w[q]);
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[j * 4 + q] = __uint_as_float(w[q]);
            }
            // groups past the end hold -inf (0xFF80 bf16 / fixed below for f32)
            if (DT == DT_F32 && j * kBlock + tid >= ngroups) {
#pragma unroll
                for (int q = 0; q < 4; ++q) v[j * 4 + q] = -INFINITY;
            }
        }
        // remainder elements (n not a multiple of `per`): fewer than `per`,
        // placed in the slots of group `ngroups`, owned by thread ngroups % 256
        const int rem = n - ngroups * per;
        if (rem > 0) {
            const int jj = ngroups / kBlock;
            if ((ngroups % kBlock) == tid && jj < nload) {
#pragma unroll
                for (int e = 0; e < per; ++e)
                    v[jj * per + e] = e < rem ? load_logit(base, DT, (long long)ngroups * per + e)
                                              : -INFINITY;
            }
        }
    } else {
        // unaligned row: element-wise loads in the same slot layout
#pragma unroll
        for (int s = 0; s < kEPT; ++s) {
            const int idx = tile_index<DT>(s);
            v[s] = idx < n ? load_logit(base, DT, idx) : -INFINITY;
        }
    }
}

// ---------------------------------------------------------------------------
// Phase A: streaming max / sum-exp over every row, one 8192-element tile per
// workgroup; the last tile of a row merges the row.
// ---------------------------------------------------------------------------
struct StreamArgs {
    Shape sh;
    float c_hi, c_lo;      // log2(e)/T split so that (x - M) * c is nearly exact
    double inv_T;
    int filtered;          // top-k or top-p active
    float* tile_m;         // [rows * nt]
    double* tile_z;
    unsigned* row_cnt;     // [rows], zero between calls
    RowRec* rec;           // [rows]
};

template <int DT>
__device__ void stream_tile(const StreamArgs& a, int row, int chunk, float& m_out, double& z_out,
                            float* s_f, double* s_d) {
    const char* rowp = row_ptr(a.sh, row);
    const int i0 = chunk * kTile;
    const int n = min(kTile, a.sh.V - i0);
    float v[kEPT];
    load_tile<DT>(rowp, i0, n, v);
    float m = v[0];
#pragma unroll
    for (int s = 1; s < kEPT; ++s) m = fmaxf(m, v[s]);
    const float M = block_max(m, s_f);
    double z = 0.0;
    if (M != -INFINITY) {
        float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < kEPT; ++s) {
            const float y = v[s] - M;
            const float t = __builtin_amdgcn_exp2f(fmaf(y, a.c_hi, y * a.c_lo));
            acc[s & 3] += t;
        }
        z = ((double)acc[0] + (double)acc[1]) + ((double)acc[2] + (double)acc[3]);
    }
    z = block_sum(z, s_d);
    m_out = M;
    z_out = z;
}

__global__ void __launch_bounds__(kBlock) k_rowstats(StreamArgs a) {
    __shared__ float s_f[kWaves];
    __shared__ double s_d[kWaves];
    __shared__ int s_last;
    const int nt = a.sh.nt;
    const long long tile = blockIdx.x;
    const int row = (int)(tile / nt);
    const int chunk = (int)(tile % nt);
    float m;
    double z;
    if (row_dt(a.sh, row) == DT_BF16)
        stream_tile<DT_BF16>(a, row, chunk, m, z, s_f, s_d);
    else
        stream_tile<DT_F32>(a, row, chunk, m, z, s_f, s_d);
    if (threadIdx.x == 0) {
        a.tile_m[tile] = m;
        a.tile_z[tile] = z;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&a.row_cnt[row], 1u) == (unsigned)(nt - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    // Merge the row: M = max tile max, Z = sum z_t * exp((m_t - M)/T) in fp64,
    // each thread over tiles tid, tid+256, ... then a fixed-order block sum.
    const size_t t0 = (size_t)row * nt;
    float mm = -INFINITY;
    for (int t = threadIdx.x; t < nt; t += kBlock) mm = fmaxf(mm, a.tile_m[t0 + t]);
    const float M = block_max(mm, s_f);
    double zz = 0.0;
    for (int t = threadIdx.x; t < nt; t += kBlock) {
        const double zt = a.tile_z[t0 + t];
        if (zt > 0.0) zz += zt * exp(((double)a.tile_m[t0 + t] - (double)M) * a.inv_T);
    }
    const double Z = block_sum(zz, s_d);
    if (threadIdx.x == 0) {
        a.row_cnt[row] = 0u;
        RowRec r;
        r.s.max_logit = M;
        r.z_all = Z;
        r.pad = 0.0;
        if (!a.filtered) {
            r.s.thresh = -INFINITY;
            r.s.n_kept = a.sh.V;
            r.s.flags = 0;
            r.s.z_kept = Z;
            double prob = __builtin_nan("");
            if (row_has_token(a.sh, row)) {
                const int d = row_token(a.sh, row);
                prob = 0.0;
                if (d >= 0 && d < a.sh.V) {
                    const float xd = load_logit(row_ptr(a.sh, row), row_dt(a.sh, row), d);
                    prob = exp(((double)xd - (double)M) * a.inv_T) / Z;
                }
            }
            r.s.prob_at_token = prob;
        } else {
            r.s.thresh = -INFINITY;
            r.s.n_kept = 0;
            r.s.flags = SPEC_ROW_FILTERED;
            r.s.z_kept = 0.0;
            r.s.prob_at_token = 0.0;
        }
        a.rec[row] = r;
    }
}

// ---------------------------------------------------------------------------
// Exact filter resolution by re-reading a row (one workgroup per row):
// radix select on order-preserving keys, 8 bits per pass, MSB first.
//   top-k: count histograms find the key of the top_k-th largest logit.
//   top-p: mass histograms (exp((x-M)/T) in fp64, summed as 64-bit fixed
//          point so that the sums are exact and order-independent) find the
//          group where the mass of strictly larger logits stops being below
//          top_p * Z.
// ---------------------------------------------------------------------------
struct ResolveArgs {
    Shape sh;
    double inv_T;
    int top_k;       // active iff 0 < top_k < V
    float top_p;     // active iff < 1
    int fx_shift;    // fixed-point scale 2^fx_shift, V * 2^fx_shift < 2^63
    RowRec* rec;
};

// Calls f(index, value) for every element of the row, threads striding over
// 16-byte groups (or single elements for unaligned rows).
template <int DT, class F>
__device__ __forceinline__ void for_each_elem(const char* rowp, int V, F&& f) {
    constexpr int esz = DT == DT_BF16 ? 2 : 4;
    constexpr int per = 16 / esz;
    if ((((uintptr_t)rowp) & 15) == 0) {
        const int ngroups = V / per;
        for (int g = threadIdx.x; g < ngroups; g += kBlock) {
            const u32x4 raw = ld16_nt(rowp + (size_t)g * 16);
            const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (DT == DT_BF16) {
                    f(g * per + 2 * q, bf16_lo(w[q]));
                    f(g * per + 2 * q + 1, bf16_hi(w[q]));
                } else {
                    f(g * per + q, __uint_as_float(w[q]));
                }
            }
        }
        for (int i = ngroups * per + threadIdx.x; i < V; i += kBlock) f(i, load_logit(rowp, DT, i));
    } else {
        for (int i = threadIdx.x; i < V; i += kBlock) f(i, load_logit(rowp, DT, i));
    }
}

// Complete a key found 16 bits at a time from a bf16 row: the low 16 bits of
// a widened bf16 are 0, so its key's low half is 0 (x >= 0) or 0xFFFF (x < 0).
__device__ __forceinline__ uint32_t bf16_key_fill(uint32_t k) {
    return (k & 0x80000000u) ? (k & 0xFFFF0000u) : (k | 0x0000FFFFu);
}

template <int DT>
__device__ void resolve_row(const ResolveArgs& a, int row) {
    __shared__ unsigned s_cnt[256];
    __shared__ unsigned long long s_mass[256];
    __shared__ uint32_t s_prefix, s_mask;
    __shared__ int s_kk;
    __shared__ unsigned long long s_A;
    __shared__ unsigned s_cabove;
    __shared__ double s_zbase;
    __shared__ unsigned long long s_zk;
    __shared__ unsigned s_nk;

    const char* rowp = row_ptr(a.sh, row);
    const int V = a.sh.V;
    const RowRec rin = a.rec[row];
    const float M = rin.s.max_logit;
    const double inv_T = a.inv_T;
    const bool use_k = a.top_k > 0 && a.top_k < V;
    const bool use_p = a.top_p < 1.0f;
    const double scale = ldexp(1.0, a.fx_shift);
    const int nlevels = DT == DT_BF16 ? 2 : 4;

    uint32_t tau_key = 0u;  // keep key >= tau_key after top-k
    if (use_k) {
        if (threadIdx.x == 0) {
            s_prefix = 0u;
            s_mask = 0u;
            s_kk = a.top_k;
        }
        for (int lvl = 0; lvl < nlevels; ++lvl) {
            const int shift = 24 - 8 * lvl;
            for (int i = threadIdx.x; i < 256; i += kBlock) s_cnt[i] = 0u;
            __syncthreads();
            const uint32_t prefix = s_prefix, mask = s_mask;
            for_each_elem<DT>(rowp, V, [&](int, float x) {
                const uint32_t k = fkey(x);
                if ((k & mask) == prefix) atomicAdd(&s_cnt[(k >> shift) & 255u], 1u);
            });
            __syncthreads();
            if (threadIdx.x == 0) {
                int kk = s_kk;
                int d = 255;
                for (; d > 0; --d) {
                    if ((int)s_cnt[d] >= kk) break;
                    kk -= (int)s_cnt[d];
                }
                s_kk = kk;
                s_prefix = prefix | ((uint32_t)d << shift);
                s_mask = mask | (0xFFu << shift);
            }
            __syncthreads();
        }
        tau_key = DT == DT_BF16 ? bf16_key_fill(s_prefix) : s_prefix;
    }

    uint32_t thr_key = tau_key;
    double z_kept = 0.0;
    unsigned n_kept = 0u;
    if (use_p) {
        if (threadIdx.x == 0) {
            s_prefix = 0u;
            s_mask = 0u;
            s_A = 0ull;
            s_cabove = 0u;
            s_zbase = rin.z_all;
        }
        for (int lvl = 0; lvl < nlevels; ++lvl) {
            const int shift = 24 - 8 * lvl;
            for (int i = threadIdx.x; i < 256; i += kBlock) {
                s_cnt[i] = 0u;
                s_mass[i] = 0ull;
            }
            __syncthreads();
            const uint32_t prefix = s_prefix, mask = s_mask;
            for_each_elem<DT>(rowp, V, [&](int, float x) {
                const uint32_t k = fkey(x);
                if (k >= tau_key && (k & mask) == prefix) {
                    const double w = exp(((double)x - (double)M) * inv_T);
                    const unsigned d = (k >> shift) & 255u;
                    atomicAdd(&s_mass[d], (unsigned long long)(w * scale));
                    atomicAdd(&s_cnt[d], 1u);
                }
            });
            __syncthreads();
            if (threadIdx.x == 0) {
                if (lvl == 0 && use_k) {
                    unsigned long long tot = 0ull;
                    for (int d = 0; d < 256; ++d) tot += s_mass[d];
                    s_zbase = (double)tot / scale;
                }
                const double zb = s_zbase;
                unsigned long long A = s_A;
                unsigned cab = s_cabove;
                int sel = -1, lowest = -1;
                unsigned long long A_low = 0ull;
                unsigned c_low = 0u;
                for (int d = 255; d >= 0; --d) {
                    if (s_cnt[d] == 0u) continue;
                    const unsigned long long incl = A + s_mass[d];
                    if (!(((double)incl / scale) / zb < (double)a.top_p)) {
                        sel = d;
                        break;
                    }
                    lowest = d;
                    A_low = A;
                    c_low = cab;
                    A = incl;
                    cab += s_cnt[d];
                }
                if (sel < 0) {  // crossing not reached (rounding): keep the whole range
                    sel = lowest;
                    A = A_low;
                    cab = c_low;
                }
                s_A = A;
                s_cabove = cab;
                s_prefix = prefix | ((uint32_t)sel << shift);
                s_mask = mask | (0xFFu << shift);
                if (lvl == nlevels - 1) {
                    s_zk = A + s_mass[sel];
                    s_nk = cab + s_cnt[sel];
                }
            }
            __syncthreads();
        }
        thr_key = DT == DT_BF16 ? bf16_key_fill(s_prefix) : s_prefix;
        z_kept = (double)s_zk / scale;
        n_kept = s_nk;
    } else if (use_k) {
        if (threadIdx.x == 0) {
            s_zk = 0ull;
            s_nk = 0u;
        }
        __syncthreads();
        unsigned long long zl = 0ull;
        unsigned nl = 0u;
        for_each_elem<DT>(rowp, V, [&](int, float x) {
            if (fkey(x) >= tau_key) {
                zl += (unsigned long long)(exp(((double)x - (double)M) * inv_T) * scale);
                ++nl;
            }
        });
        atomicAdd(&s_zk, zl);
        atomicAdd(&s_nk, nl);
        __syncthreads();
        z_kept = (double)s_zk / scale;
        n_kept = s_nk;
    }

    if (threadIdx.x == 0) {
        RowRec r = rin;
        const float thr = key_to_float(thr_key);
        r.s.thresh = thr;
        r.s.n_kept = (int)n_kept;
        r.s.flags = SPEC_ROW_FILTERED | SPEC_ROW_EXACT_PATH;
        r.s.z_kept = z_kept;
        double prob = __builtin_nan("");
        if (row_has_token(a.sh, row)) {
            const int d = row_token(a.sh, row);
            prob = 0.0;
            if (d >= 0 && d < V) {
                const float xd = load_logit(rowp, DT, d);
                if (xd >= thr) prob = exp(((double)xd - (double)M) * inv_T) / z_kept;
            }
        }
        r.s.prob_at_token = prob;
        a.rec[row] = r;
    }
}

__global__ void __launch_bounds__(kBlock) k_resolve(ResolveArgs a) {
    const int row = blockIdx.x;
    if (row_dt(a.sh, row) == DT_BF16)
        resolve_row<DT_BF16>(a, row);
    else
        resolve_row<DT_F32>(a, row);
}

// ---------------------------------------------------------------------------
// Phases B and C: accept scan and the stop-token draw.
// Grid: B * n_chunks workgroups; workgroup (b, c) finds the stop position j of
// sequence b (every workgroup of b recomputes it: K probabilities and K
// Philox blocks), sums the residual (and p_j) over chunk c of the stop row in
// fp64, and the last workgroup of b to finish locates the inverse-CDF point.
// ---------------------------------------------------------------------------
constexpr int kChunk = 8192;              // elements per sampling chunk
constexpr int kCPT = kChunk / kBlock;     // 32 contiguous elements per thread

struct SampleArgs {
    Shape sh;
    double inv_T;
    uint64_t seed;
    int n_chunks;
    const RowRec* rec;
    double2* chunk_sum;   // [B * n_chunks] (.x residual, .y p)
    unsigned* seq_cnt;    // [B], zero between calls
    int32_t* out_tokens;
    int32_t* out_num;
};

// Stop position of sequence b, computed by one wave (all lanes return it).
__device__ __forceinline__ int first_rejection(const SampleArgs& a, int b) {
    const int lane = threadIdx.x & 63;
    const int K = a.sh.K;
    for (int k0 = 0; k0 < K; k0 += 64) {
        const int k = k0 + lane;
        bool reject = false;
        if (k < K) {
            const double p = a.rec[(size_t)b * (K + 1) + k].s.prob_at_token;
            const double q = a.rec[a.sh.n_trows + (size_t)b * K + k].s.prob_at_token;
            const double u = uniform24(draw_block(a.seed, (uint32_t)b, (uint32_t)k, PURPOSE_ACCEPT));
            reject = !(u * q < p);
        }
        const unsigned long long m = __ballot(reject);
        if (m) return k0 + __ffsll((long long)m) - 1;
    }
    return K;
}

struct StopRow {
    const char* tp; const char* dp;
    int tdt, ddt;
    float Mt, Md, thr_t, thr_d;
    double zt, zd;
    bool has_draft;
};

// p_j(i) and the residual max(0, p_j(i) - q_j(i)) for one token, fp64.
__device__ __forceinline__ void stop_terms(const StopRow& s, double inv_T, int i, double& p, double& r) {
    const float xt = load_logit(s.tp, s.tdt, i);
    p = xt >= s.thr_t ? exp(((double)xt - (double)s.Mt) * inv_T) / s.zt : 0.0;
    double q = 0.0;
    if (s.has_draft) {
        const float xd = load_logit(s.dp, s.ddt, i);
        q = xd >= s.thr_d ? exp(((double)xd - (double)s.Md) * inv_T) / s.zd : 0.0;
    }
    const double d = p - q;
    r = d > 0.0 ? d : 0.0;
}

// Deterministic exclusive scan of one double per thread (thread order),
// also returning the total.  Same code for chunk totals and for the search,
// so both see identical prefixes.
__device__ void block_excl_scan(double v, double* s_val, double* s_excl, double& excl, double& total) {
    __shared__ double s_total;
    const int tid = threadIdx.x;
    s_val[tid] = v;
    __syncthreads();
    if (tid < 64) {
        const double v0 = s_val[4 * tid], v1 = s_val[4 * tid + 1];
        const double v2 = s_val[4 * tid + 2], v3 = s_val[4 * tid + 3];
        const double ls = ((v0 + v1) + v2) + v3;
        double incl = ls;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
            const double t = __shfl_up(incl, off, 64);
            if (tid >= off) incl += t;
        }
        double e = __shfl_up(incl, 1, 64);
        if (tid == 0) e = 0.0;
        s_excl[4 * tid] = e;
        e += v0;
        s_excl[4 * tid + 1] = e;
        e += v1;
        s_excl[4 * tid + 2] = e;
        e += v2;
        s_excl[4 * tid + 3] = e;
        if (tid == 63) s_total = incl;
    }
    __syncthreads();
    excl = s_excl[tid];
    total = s_total;
    __syncthreads();
}

__global__ void __launch_bounds__(kBlock) k_sample(SampleArgs a) {
    __shared__ int s_j;
    __shared__ int s_last;
    __shared__ double s_val[kBlock];
    __shared__ double s_excl[kBlock];
    __shared__ int s_cstar;
    __shared__ double s_run, s_t;
    __shared__ int s_usep;
    __shared__ int s_tau;
    const int b = blockIdx.x / a.n_chunks;
    const int c = blockIdx.x % a.n_chunks;
    const int K = a.sh.K, V = a.sh.V;

    if (threadIdx.x < 64) {
        const int j = first_rejection(a, b);
        if (threadIdx.x == 0) s_j = j;
    }
    __syncthreads();
    const int j = s_j;

    StopRow s;
    const int rt = b * (K + 1) + j;
    const RowRec& Rt = a.rec[rt];
    s.tp = row_ptr(a.sh, rt);
    s.tdt = a.sh.tdt;
    s.Mt = Rt.s.max_logit;
    s.thr_t = Rt.s.thresh;
    s.zt = Rt.s.z_kept;
    s.has_draft = j < K;
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

    // chunk sums over this thread's 32 contiguous tokens, then block totals
    {
        const int lo = c * kChunk + threadIdx.x * kCPT;
        const int hi = min(lo + kCPT, V);
        double sr = 0.0, sp = 0.0;
        for (int i = lo; i < hi; ++i) {
            double p, r;
            stop_terms(s, a.inv_T, i, p, r);
            sr += r;
            sp += p;
        }
        double e, tr, tp;
        block_excl_scan(sr, s_val, s_excl, e, tr);
        block_excl_scan(sp, s_val, s_excl, e, tp);
        if (threadIdx.x == 0) a.chunk_sum[(size_t)b * a.n_chunks + c] = make_double2(tr, tp);
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        s_last = (atomicAdd(&a.seq_cnt[b], 1u) == (unsigned)(a.n_chunks - 1));
    __syncthreads();
    if (!s_last) return;
    __threadfence();

    if (threadIdx.x == 0) {
        a.seq_cnt[b] = 0u;
        const double2* cs = a.chunk_sum + (size_t)b * a.n_chunks;
        double Sr = 0.0, Sp = 0.0;
        for (int cc = 0; cc < a.n_chunks; ++cc) {
            const double2 v = cs[cc];
            Sr += v.x;
            Sp += v.y;
        }
        const int usep = (j == K) || !(Sr > 0.0);
        const double S = usep ? Sp : Sr;
        const double t = uniform53(draw_block(a.seed, (uint32_t)b, (uint32_t)j, PURPOSE_SAMPLE)) * S;
        double run = 0.0;
        int cstar = -1, last_nz = -1;
        double run_last = 0.0;
        for (int cc = 0; cc < a.n_chunks; ++cc) {
            const double2 v = cs[cc];
            const double sc = usep ? v.y : v.x;
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
        if (cstar < 0) {  // t at or past the total after rounding
            cstar = last_nz;
            run = run_last;
        }
        s_cstar = cstar;
        s_run = run;
        s_t = t;
        s_usep = usep;
    }
    __syncthreads();
    const int cstar = s_cstar;
    const double run = s_run, t = s_t;
    const bool usep = s_usep != 0;

    // recompute this thread's sums on chunk c*, scan, pick the thread range
    const int lo = cstar * kChunk + threadIdx.x * kCPT;
    const int hi = min(lo + kCPT, V);
    double sr = 0.0, sp = 0.0;
    for (int i = lo; i < hi; ++i) {
        double p, r;
        stop_terms(s, a.inv_T, i, p, r);
        sr += r;
        sp += p;
    }
    const double mine = usep ? sp : sr;
    double excl, total;
    block_excl_scan(mine, s_val, s_excl, excl, total);
    // largest thread with mass whose range starts at or before t
    if (threadIdx.x == 0) s_tau = -1;
    __syncthreads();
    if (mine > 0.0 && run + excl <= t) atomicMax(&s_tau, (int)threadIdx.x);
    __syncthreads();
    if (s_tau < 0) {  // every positive range starts after t: first positive one
        if (threadIdx.x == 0) s_tau = kBlock;
        __syncthreads();
        if (mine > 0.0) atomicMin(&s_tau, (int)threadIdx.x);
        __syncthreads();
    }
    if ((int)threadIdx.x == s_tau) {
        double acc = run + excl;
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
        if (y < 0) y = last;
        int32_t* out = a.out_tokens + (size_t)b * (K + 1);
        for (int k = 0; k < j; ++k) out[k] = a.sh.tokens[(size_t)b * K + k];
        out[j] = y;
        for (int k = j + 1; k <= K; ++k) out[k] = -1;
        a.out_num[b] = j;
    }
}

// Copy row records to the caller's stats arrays.
__global__ void k_copy_stats(const RowRec* rec, int n_trows, int n_drows,
                             spec_row_stats_t* tstats, spec_row_stats_t* dstats) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n_trows) {
        if (tstats) tstats[i] = rec[i].s;
    } else if (i < n_trows + n_drows) {
        if (dstats) dstats[i - n_trows] = rec[i].s;
    }
}

// ---------------------------------------------------------------------------
// Greedy: argmax per target row (lowest index on ties) with packed 64-bit
// keys (order-preserving value key << 32 | ~index) merged by atomicMax; the
// last tile of a sequence matches the prefix and writes the outputs.
// ---------------------------------------------------------------------------
struct GreedyArgs {
    Shape sh;              // draft fields unused
    unsigned long long* gkey;  // [B*(K+1)], zero between calls
    unsigned* seq_cnt;     // [B], zero between calls
    int32_t* out_tokens;
    int32_t* out_num;
};

template <int DT>
__device__ __forceinline__ unsigned long long greedy_tile(const GreedyArgs& a, int row, int chunk) {
    const char* rowp = row_ptr(a.sh, row);
    const int i0 = chunk * kTile;
    const int n = min(kTile, a.sh.V - i0);
    float v[kEPT];
    load_tile<DT>(rowp, i0, n, v);
    // thread-local first maximum over valid slots (slots are in increasing
    // index order within a thread)
    float best = -INFINITY;
    int bidx = -1;
#pragma unroll
    for (int s = 0; s < kEPT; ++s) {
        const int idx = tile_index<DT>(s);
        if (idx < n && (bidx < 0 || v[s] > best)) {
            best = v[s];
            bidx = idx;
        }
    }
    unsigned long long key = 0ull;
    if (bidx >= 0)
        key = ((unsigned long long)fkey(best) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)(i0 + bidx));
    return wave_max_u64(key);
}

__global__ void __launch_bounds__(kBlock) k_greedy(GreedyArgs a) {
    __shared__ unsigned long long s_k[kWaves];
    __shared__ int s_last;
    const int nt = a.sh.nt;
    const long long tile = blockIdx.x;
    const int row = (int)(tile / nt);
    const int chunk = (int)(tile % nt);
    const unsigned long long wk =
        a.sh.tdt == DT_BF16 ? greedy_tile<DT_BF16>(a, row, chunk) : greedy_tile<DT_F32>(a, row, chunk);
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    if (lane == 0) s_k[wid] = wk;
    __syncthreads();
    const int K = a.sh.K;
    const int b = row / (K + 1);
    if (threadIdx.x == 0) {
        unsigned long long k = s_k[0];
        for (int w = 1; w < kWaves; ++w) k = s_k[w] > k ? s_k[w] : k;
        atomicMax(&a.gkey[row], k);
        __threadfence();
        s_last = (atomicAdd(&a.seq_cnt[b], 1u) == (unsigned)((K + 1) * nt - 1));
    }
    __syncthreads();
    if (!s_last || threadIdx.x != 0) return;
    __threadfence();
    a.seq_cnt[b] = 0u;
    unsigned long long* slots = a.gkey + (size_t)b * (K + 1);
    // argmax index of target row k (reads are atomic: the slots were written
    // by atomics from other workgroups)
    auto g_of = [&](int k) {
        const unsigned long long key = __hip_atomic_load(&slots[k], __ATOMIC_RELAXED,
                                                         __HIP_MEMORY_SCOPE_AGENT);
        return (int)(0xFFFFFFFFu - (uint32_t)(key & 0xFFFFFFFFull));
    };
    int j = K;
    for (int k = 0; k < K; ++k)
        if (a.sh.tokens[(size_t)b * K + k] != g_of(k)) {
            j = k;
            break;
        }
    int32_t* out = a.out_tokens + (size_t)b * (K + 1);
    for (int k = 0; k < j; ++k) out[k] = a.sh.tokens[(size_t)b * K + k];
    out[j] = g_of(j);
    for (int k = j + 1; k <= K; ++k) out[k] = -1;
    a.out_num[b] = j;
    for (int k = 0; k <= K; ++k) slots[k] = 0ull;  // zero for the next call
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
