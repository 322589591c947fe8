// row_kernels.h — per-row kernels: one 512-thread workgroup streams one whole
// logit row from HBM exactly once.
//
//  k_row     : sampling mode.  Three row modes:
//                plain   (no filter)      running max / sum of exp((x-M)/T);
//                nucleus (top-p only)     the same sums, plus candidate capture;
//                top-k   (top-k active)   candidate capture only: the kept set
//                                         and its mass come from the top-k
//                                         candidates, so no sum over the row.
//              Capture: every 16-byte load (8 bf16 or 4 fp32 logits) whose
//              maximum reaches a threshold set from the row's first tile is
//              appended, raw, to its wave's LDS segment, and expanded 64
//              units at a time into (logit, index) candidates while the row
//              streams.  After the stream the kept set is resolved exactly
//              from the candidates and, if they cannot decide (overflow, too
//              few), by re-reading the row.  Writes the row record (M, Z,
//              threshold, p(d_k) or q(d_k)) and, for target rows of drafted
//              sequences, the kept tokens sorted by index (token trees draw
//              from the stop row itself and skip the lists).
//  k_row_argmax : greedy mode, lowest-index argmax of a target row.
//
// Row numbering: rows [0, B*(K+1)) are target rows b*(K+1)+k, rows
// [B*(K+1), B*(2K+1)) are draft rows b*K+k (none for point-mass drafts; for
// a token tree K is the node count and target row k+1 follows node k).
// With per-sequence draft lengths, rows past a sequence's length exit at once.
// Workgroup i takes row i, or, when rows outnumber what the GPU runs at once,
// the draft rows first (k_row).
#pragma once

#include <type_traits>

#include "device_common.h"
#include "../../include/spec_verify.h"

namespace sv {

typedef unsigned long long u64;

constexpr int kRB = 512;                 // threads per row workgroup
constexpr int kRW = kRB / 64;            // waves per row workgroup
constexpr int kREPT = 16;                // logits per thread per tile
constexpr int kRTile = kRB * kREPT;      // 8192 logits per tile
constexpr int kSegU = 256;               // captured 16-byte units per wave segment
constexpr int kUnits = kSegU * kRW;      // 2048 units per workgroup
constexpr int kCW = 320;                 // candidates (logit, index) per wave after expansion
constexpr int kCap = kCW * kRW;          // candidates per workgroup (2560)
constexpr int kOwn = (kCW + 63) / 64;    // candidates per thread during resolution (5)
constexpr int kR0 = 64;                  // rank among thread maxima for the first threshold
constexpr int kListMax = 4096;           // longest kept list stored for the draw

enum { MODE_PLAIN = 0, MODE_NUCLEUS = 1, MODE_TOPK = 2 };

constexpr int kBufWord3 = 0x00020000;    // raw buffer descriptor, word 3, for gfx9-family parts
constexpr int kLoadNT = 2;               // cache policy of streaming loads: non-temporal

struct RowRec {
    spec_row_stats_t s;
    double z_all;  // sum over all tokens of exp((x - M)/T), before filters
    double pad;
};
static_assert(sizeof(spec_row_stats_t) == 32, "row stats layout");

struct Shape {
    const char* target;
    const char* draft;
    const int32_t* tokens;
    int B, K, V;
    int tdt, ddt;
    int tsz, dsz;
    int n_trows, n_drows;
    const int32_t* lens;  // per-sequence draft lengths in [0, K] (clamped), or null: all K
    int32_t* tested;      // [K] per-position acceptance counters, each may be null (zeroed by
    int32_t* accepted;    //   the row kernel's first workgroup, counted by the output writers)
};

// The first row workgroup of a call clears the acceptance counters; the
// kernels that write a sequence's outputs run after it on the stream.
__device__ __forceinline__ void clear_counters(const Shape& sh) {
    if (blockIdx.x != 0) return;
    for (int k = threadIdx.x; k < sh.K; k += blockDim.x) {
        if (sh.tested) sh.tested[k] = 0;
        if (sh.accepted) sh.accepted[k] = 0;
    }
}

__device__ __forceinline__ const char* row_ptr(const Shape& sh, int row) {
    if (row < sh.n_trows) return sh.target + (size_t)row * sh.V * sh.tsz;
    return sh.draft + (size_t)(row - sh.n_trows) * sh.V * sh.dsz;
}
__device__ __forceinline__ int row_dt(const Shape& sh, int row) {
    return row < sh.n_trows ? sh.tdt : sh.ddt;
}
// Draft length of sequence b: its first K_b drafts are verified against
// target rows 0..K_b (the bonus comes from row K_b); rows past them are not
// read.
__device__ __forceinline__ int seq_len(const Shape& sh, int b) {
    return sh.lens ? min(max(sh.lens[b], 0), sh.K) : sh.K;
}
__device__ __forceinline__ bool row_live(const Shape& sh, int row) {
    if (!sh.lens) return true;
    if (row < sh.n_trows) return row % (sh.K + 1) <= seq_len(sh, row / (sh.K + 1));
    const int r = row - sh.n_trows;
    return r % sh.K < seq_len(sh, r / sh.K);
}
// Rows of a token tree carry no token of their own (tokens is null there).
__device__ __forceinline__ bool row_has_token(const Shape& sh, int row) {
    return sh.tokens && (row >= sh.n_trows || (row % (sh.K + 1)) < seq_len(sh, row / (sh.K + 1)));
}
__device__ __forceinline__ int row_token(const Shape& sh, int row) {
    if (row < sh.n_trows) {
        const int b = row / (sh.K + 1), k = row % (sh.K + 1);
        return sh.tokens[(size_t)b * sh.K + k];
    }
    return sh.tokens[row - sh.n_trows];
}

// ---------------------------------------------------------------------------
// Block helpers for kRB threads (fixed combination order: deterministic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float rb_max(float v, float* s) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = s[0];
#pragma unroll
    for (int w = 1; w < kRW; ++w) r = fmaxf(r, s[w]);
    return r;
}
__device__ __forceinline__ double rb_sum(double v, double* s) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = s[0];
#pragma unroll
    for (int w = 1; w < kRW; ++w) r += s[w];
    return r;
}
__device__ __forceinline__ u64 wave_sum_u64(u64 v) {
    return wave_allreduce(v, [](u64 a, u64 b) { return a + b; });
}
__device__ __forceinline__ u64 rb_sum_u64(u64 v, u64* s) {
    v = wave_sum_u64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    u64 r = 0;
#pragma unroll
    for (int w = 0; w < kRW; ++w) r += s[w];
    return r;
}
__device__ __forceinline__ u64 rb_max_u64(u64 v, u64* s) {
    v = wave_max_u64(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = v;
    __syncthreads();
    u64 r = s[0];
#pragma unroll
    for (int w = 1; w < kRW; ++w) r = s[w] > r ? s[w] : r;
    return r;
}

// One wave scans 256 histogram bins from bin 255 down and returns the first
// bin d where (sum of bins above d) + hist[d] >= target, with the sum above d.
// bin = -1 when the total stays below target (then above = total).
__device__ __forceinline__ void wave_find_from_top(const u64* hist, u64 target, int& bin, u64& above) {
    const int lane = threadIdx.x & 63;
    u64 c[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) c[i] = hist[255 - 4 * lane - i];
    const u64 ls = c[0] + c[1] + c[2] + c[3];
    const u64 incl = wave_incl_scan(ls);
    const u64 excl = incl - ls;
    const u64 m = __ballot(incl >= target);
    if (m == 0) {
        bin = -1;
        above = lane_read(incl, 63);
        return;
    }
    const int L = __ffsll((long long)m) - 1;
    int d = 0;
    u64 run = excl;
    if (lane == L) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (run + c[i] >= target) {
                d = 255 - 4 * lane - i;
                break;
            }
            run += c[i];
        }
    }
    bin = lane_read(d, L);
    above = lane_read(run, L);
}

// Result of a block-wide selection from the top.
struct Sel {
    uint32_t key;     // selected group (exact key)
    u64 above;        // weight of entries with a larger key
    u64 group;        // weight of the selected group
    uint32_t cnt_above, cnt_group;
    int ok;           // 0: the total weight stays below the target
};

// Complete a key known in its top 16 bits, for widened bf16 values whose low
// 16 bits are zero: key low half is 0 for x >= 0 and 0xFFFF for x < 0.
__device__ __forceinline__ uint32_t bf16_key_fill(uint32_t k) {
    return (k & 0x80000000u) ? (k & 0xFFFF0000u) : (k | 0x0000FFFFu);
}

// ---------------------------------------------------------------------------
// Row streaming: 16-byte non-temporal loads, groups g = t*kRB*NL + j*kRB + tid
// (each load instruction of the workgroup covers 8 KiB contiguous).  The
// logit at slot s = j*per + q of tile t has index per*g + q.  Groups past the
// end, the partial last group and unaligned rows use element loads.
// ---------------------------------------------------------------------------
template <int DT>
struct RowStream {
    static constexpr int esz = DT == DT_BF16 ? 2 : 4;
    static constexpr int per = 16 / esz;
    static constexpr int NL = kREPT / per;  // 16-byte loads per thread per tile
    const char* rowp;
    int V;
    int gfull;     // groups that can be read with one 16-byte load
    int nt;        // tiles
    int nfull;     // leading tiles whose every group is a full 16-byte load
    __amdgpu_buffer_rsrc_t rsrc;  // the row as a raw buffer

    __device__ RowStream(const char* p, int v) : rowp(p), V(v) {
        const bool aligned = (((uintptr_t)p) & 15) == 0;
        gfull = aligned ? V / per : 0;
        const int ng = (V + per - 1) / per;
        nt = (ng + kRB * NL - 1) / (kRB * NL);
        nfull = gfull / (kRB * NL);
        rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(p), 0, V * esz, kBufWord3);
    }
    __device__ __forceinline__ int group(int t, int j) const {
        return t * kRB * NL + j * kRB + (int)threadIdx.x;
    }
    __device__ __forceinline__ int index(int t, int s) const {
        return group(t, s / per) * per + s % per;
    }
    // tile t < nfull: every load in bounds, no checks.  The tile and load
    // offsets are uniform (scalar offset), the lane's offset is the same for
    // every load, so no per-load address arithmetic.
    __device__ __forceinline__ void issue_full(int t, u32x4 (&raw)[NL]) const {
#pragma unroll
        for (int j = 0; j < NL; ++j)
            raw[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                   rsrc, (int)(threadIdx.x * 16u), (t * NL + j) * (kRB * 16),
                                                   kLoadNT));
    }
    // any tile: groups past the full ones load group 0 instead (needs gfull > 0)
    __device__ __forceinline__ void issue_clamped(int t, u32x4 (&raw)[NL]) const {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int g = group(t, j);
            raw[j] = ld16_nt(rowp + (size_t)(g < gfull ? g : 0) * 16);
        }
    }
    __device__ __forceinline__ void issue(int t, u32x4 (&raw)[NL]) const {
        if (t < nfull) {
            issue_full(t, raw);
            return;
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int g = group(t, j);
            if (g < gfull) raw[j] = ld16_nt(rowp + (size_t)g * 16);
        }
    }
    __device__ __forceinline__ static void unpack_full(const u32x4 (&raw)[NL], float (&v)[kREPT]) {
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                if (DT == DT_BF16) {
                    v[j * 8 + 2 * q] = bf16_lo(w[q]);
                    v[j * 8 + 2 * q + 1] = bf16_hi(w[q]);
                } else {
                    v[j * 4 + q] = __uint_as_float(w[q]);
                }
            }
        }
    }
    __device__ __forceinline__ void unpack(int t, const u32x4 (&raw)[NL], float (&v)[kREPT]) const {
        if (t < nfull) {
            unpack_full(raw, v);
            return;
        }
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            const int g = group(t, j);
            if (g < gfull) {
                const uint32_t w[4] = {raw[j].x, raw[j].y, raw[j].z, raw[j].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (DT == DT_BF16) {
                        v[j * 8 + 2 * q] = bf16_lo(w[q]);
                        v[j * 8 + 2 * q + 1] = bf16_hi(w[q]);
                    } else {
                        v[j * 4 + q] = __uint_as_float(w[q]);
                    }
                }
            } else {
#pragma unroll
                for (int q = 0; q < per; ++q) {
                    const int idx = g * per + q;
                    v[j * per + q] = idx < V ? load_logit(rowp, DT, idx) : -INFINITY;
                }
            }
        }
    }
    // Group j of a tile in its stored 16-byte form, rebuilt from the widened
    // values (slots past the end of the row hold -inf).
    __device__ __forceinline__ static u32x4 repack(const float (&v)[kREPT], int j) {
        u32x4 u;
        if (DT == DT_BF16) {
            u.x = (__float_as_uint(v[j * 8 + 1]) & 0xFFFF0000u) | (__float_as_uint(v[j * 8 + 0]) >> 16);
            u.y = (__float_as_uint(v[j * 8 + 3]) & 0xFFFF0000u) | (__float_as_uint(v[j * 8 + 2]) >> 16);
            u.z = (__float_as_uint(v[j * 8 + 5]) & 0xFFFF0000u) | (__float_as_uint(v[j * 8 + 4]) >> 16);
            u.w = (__float_as_uint(v[j * 8 + 7]) & 0xFFFF0000u) | (__float_as_uint(v[j * 8 + 6]) >> 16);
        } else {
            u.x = __float_as_uint(v[j * 4 + 0]);
            u.y = __float_as_uint(v[j * 4 + 1]);
            u.z = __float_as_uint(v[j * 4 + 2]);
            u.w = __float_as_uint(v[j * 4 + 3]);
        }
        return u;
    }
    // Logit q of a stored 16-byte group, widened.
    __device__ __forceinline__ static float unit_value(const u32x4& u, int q) {
        if (DT == DT_BF16) {
            const uint32_t w = (q >> 1) == 0 ? u.x : (q >> 1) == 1 ? u.y : (q >> 1) == 2 ? u.z : u.w;
            return (q & 1) ? bf16_hi(w) : bf16_lo(w);
        }
        return __uint_as_float(q == 0 ? u.x : q == 1 ? u.y : q == 2 ? u.z : u.w);
    }
};

// ---------------------------------------------------------------------------
// k_row
// ---------------------------------------------------------------------------
constexpr int kNB = 512;                 // value bins used to resolve filters
constexpr int kBinMax = 512;             // largest bin resolved pairwise

// Streaming statistics of one part of a row (rows split across workgroups).
struct PartRec {
    float m, k;  // maximum, power-of-two reference
    double z;    // sum of 2^(x c - 8 k) over the part
};
constexpr int kPartTiles = 4;             // tiles of one part, loaded together
constexpr int kMaxParts = 16;             // parts of one row at most
constexpr int kSplitRows = 512;           // rows are split only when fewer than this

struct RowArgs {
    Shape sh;
    float c_hi, c_lo;   // log2(e)/T = c_hi + c_lo to about 2^-48 relative, c_hi < log2(e)/T, c_lo > 0
    double c64;         // log2(e)/T
    float c8;           // log2(e)/(8 T), rounded
    double inv_T;
    int top_k;          // active iff use_k
    float top_p;        // active iff use_p
    int use_k, use_p;
    int fx_shift;       // fixed-point scale 2^fx_shift for weights <= 1
    RowRec* rec;
    uint2* kept;        // [n_trows][kListMax] (index, logit bits), ascending index
    int* kept_n;        // [n_trows]; -1 when the list was not stored
    float* kept_d;      // [n_trows][kListMax] draft logit of each listed token (rows with a draft row)
    double* kept_p;     // [n_trows][kListMax] p of each listed token
    int want_list;      // target rows store their kept lists (else the draw reads the row itself)
    int drafts_first;   // draft rows take the first workgroups (see k_row)
    int parts;          // > 1: unfiltered rows split into this many parts (one workgroup each)
    PartRec* prec;      // [rows][parts]
    unsigned* part_cnt; // [kSplitRows * kCntStride] arrival counters of the parts (zero between calls)
    unsigned* draw_cnt; // [n_cnt * kCntStride] arrival counters of the draw kernel, cleared by the first workgroup
    int n_cnt;
};

struct RowShared {
    union {
        struct {                      // while the row streams: one segment per wave
            u32x4 raw[kUnits + 64];   // captured 16-byte groups, as stored (+ a scratch slot per lane)
            uint32_t grp[kUnits + 64];  // their group numbers
        } st;
        u64 list[kListMax];           // after every wave expanded its segment: the kept list
    } u;
    u64 cand[kCap + 64];      // per-wave candidates (logit bits << 32) | index (+ a scratch slot per lane)
    u64 hm[kNB];              // per-bin fixed-point mass
    uint32_t hc[kNB];         // per-bin count
    uint32_t bkey[kBinMax];   // entries of one bin
    u64 bw[kBinMax];
    uint32_t th_hc[kNB];      // histogram of the first threshold
    Sel sel;
    double red_d[kRW];
    float red_f[kRW];
    u64 red_u[kRW];
    int red_i[kRW];
    uint32_t red_k[kRW];
    double tot_z[kRW];        // the row totals, per wave (one exchange per workgroup)
    u64 tot_c[kRW];
    float tot_m[kRW];
    float tot_k[kRW];
    int nbin;
    int nbin2[2];             // gather counters of the two bin resolutions
    int nlist;
    int ibin;
    u64 bc_u[2];              // results handed from wave 0 to the others
    u64 bc_m;
    double side_zs;           // wave 1's side results of the resolution
    double side_pt;
    uint32_t bc_k[2];
    int bc_i;
    u64 ubefore;
    uint32_t cbefore;
};

__device__ __forceinline__ float rb_min(float v, float* s) { return -rb_max(-v, s); }

// Exclusive prefix of one int per thread in thread order; also the total.
__device__ __forceinline__ int rb_excl_scan(int v, int* s, int& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int incl = wave_incl_scan(v);
    __syncthreads();
    if (lane == 63) s[wave] = incl;
    __syncthreads();
    int before = 0;
    total = 0;
#pragma unroll
    for (int w = 0; w < kRW; ++w) {
        before += w < wave ? s[w] : 0;
        total += s[w];
    }
    return before + incl - v;
}

// Block-wide (sum, sum, min) of a count, a mass and a key, in one exchange.
__device__ __forceinline__ void rb_count_mass_min(uint32_t& c, u64& m, uint32_t& k, RowShared& S) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    c = wave_allreduce(c, [](uint32_t a, uint32_t b) { return a + b; });
    m = wave_allreduce(m, [](u64 a, u64 b) { return a + b; });
    k = wave_allreduce(k, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
    __syncthreads();
    if (lane == 0) {
        S.red_i[wave] = (int)c;
        S.red_u[wave] = m;
        S.red_k[wave] = k;
    }
    __syncthreads();
    c = 0u;
    m = 0ull;
    k = 0xFFFFFFFFu;
#pragma unroll
    for (int w = 0; w < kRW; ++w) {
        c += (uint32_t)S.red_i[w];
        m += S.red_u[w];
        k = min(k, S.red_k[w]);
    }
}

// A wave scans bins 0..kNB-1 in order and finds the first bin at
// which the running sum of va(b) reaches target; returns it with the sums of
// va and vb over the bins before it (bin = -1 and the totals when target is
// never reached).
template <class FA, class FB>
__device__ __forceinline__ void wave_first_reach(FA&& va, FB&& vb, u64 target, int& bin, u64& before_a,
                                                 u64& before_b) {
    constexpr int per = kNB / 64;
    const int lane = threadIdx.x & 63;
    u64 c[per], d[per];
    u64 la = 0ull, lb = 0ull;
#pragma unroll
    for (int i = 0; i < per; ++i) {
        c[i] = va(per * lane + i);
        d[i] = vb(per * lane + i);
        la += c[i];
        lb += d[i];
    }
    const u64 ia = wave_incl_scan(la), ib = wave_incl_scan(lb);
    const u64 m = __ballot(ia >= target);
    if (m == 0) {
        bin = -1;
        before_a = lane_read(ia, 63);
        before_b = lane_read(ib, 63);
        return;
    }
    const int L = __ffsll((long long)m) - 1;
    int dbin = 0;
    u64 ra = ia - la, rb = ib - lb;
    if (lane == L) {
#pragma unroll
        for (int i = 0; i < per; ++i) {
            if (ra + c[i] >= target) {
                dbin = per * lane + i;
                break;
            }
            ra += c[i];
            rb += d[i];
        }
    }
    bin = lane_read(dbin, L);
    before_a = lane_read(ra, L);
    before_b = lane_read(rb, L);
}

// Capture for one tile.  Every wave owns a segment of kSegU slots and a
// uniform fill count (a scalar register).  The ballots of the tile's loads
// are taken first; if they all fit, the lanes whose group maximum reaches tau
// store their 16 bytes and group number at fill + (rank among the hits),
// otherwise the segment stops growing and ovf is raised.  No atomics, no
// branches and no exec-mask changes.
template <int NL>
__device__ __forceinline__ void capture_units(RowShared& S, const u32x4 (&unit)[NL], const float (&gm)[NL],
                                              int gbase, int gstride, float tau, int& fill, int& ovf) {
    const int seg0 = (threadIdx.x >> 6) * kSegU;
    u64 m[NL];
    int c[NL];
    int tot = 0;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        m[j] = __builtin_amdgcn_ballot_w64(gm[j] >= tau);
        c[j] = __popcll(m[j]);
        tot += c[j];
    }
    const bool ok = fill + tot <= kSegU;
    const int lane = threadIdx.x & 63;
    int f = fill;
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        // lanes without a hit (or all lanes once the segment is full) store
        // into their own scratch slot past the segments, so every lane
        // stores and nothing branches
        const int r = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m[j] >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m[j], 0u));
        const int mine = (ok && gm[j] >= tau) ? 1 : 0;
        const int pos = kUnits + lane + mine * (seg0 + f + r - kUnits - lane);
        S.u.st.raw[pos] = unit[j];
        S.u.st.grp[pos] = (uint32_t)(gbase + j * gstride);
        f += c[j];
    }
    fill = __builtin_amdgcn_readfirstlane(ok ? f : fill);
    ovf = __builtin_amdgcn_readfirstlane(ok ? ovf : 1);
}

// Expands the units [from, min(from + 64, fill)) of this wave's segment into
// candidates, every logit >= tau of every captured group, as (logit bits <<
// 32) | index, appended in segment order (one unit per lane, lane order is
// ascending token index) to the wave's own region S.cand[wave * kCW, ...)
// after its first `base` entries.  Candidates past kCW, and the values that
// are no candidates, go to the lane's scratch slot, so nothing branches per
// lane.  Returns the wave's candidate count (uniform, base included) with bit
// 32 set when the segment or the region overflowed.
template <int DT>
__device__ __forceinline__ u64 wave_expand(RowShared& S, int V, float tau, int from, int fill, int ovf, int base) {
    constexpr int per = RowStream<DT>::per;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    u64* region = S.cand + wave * kCW;
    // a slot past the fill holds stale bytes and counts no hits
    const int k = wave * kSegU + min(from + lane, kSegU - 1);
    const u32x4 ur = S.u.st.raw[k];
    const uint32_t ug = S.u.st.grp[k];
    const int lim = from + lane < fill ? V - (int)ug * per : 0;  // slots of the unit inside the row
    int c = 0;
#pragma unroll
    for (int q = 0; q < per; ++q) c += (q < lim && RowStream<DT>::unit_value(ur, q) >= tau) ? 1 : 0;
    const int incl = wave_incl_scan(c);
    const int n = base + lane_read(incl, 63);
    int p = base + incl - c;
#pragma unroll
    for (int q = 0; q < per; ++q) {
        const float x = RowStream<DT>::unit_value(ur, q);
        const bool hit = q < lim && x >= tau;
        u64* slot = (hit && p < kCW) ? region + p : S.cand + kCap + lane;
        *slot = ((u64)__float_as_uint(x) << 32) | (ug * per + q);
        p += hit ? 1 : 0;
    }
    return (u64)min(n, kCW) | ((u64)((n > kCW ? 1 : 0) | ovf) << 32);
}

// A row's totals: the largest logit, the per-thread sums taken to the
// largest grid reference k (exact power-of-two rescales) and added, and the
// sum of one 64-bit count per wave (lane 0's).  Inside a wave: the maxima
// first, then every sum rescaled to the wave's k and added in a fixed
// pattern; across waves the same in wave order, so the result does not
// depend on timing.  One barrier, on slots of its own: at most one call per
// workgroup.
struct RowTot {
    float m, k;
    double z;
    u64 c;
};
__device__ __forceinline__ RowTot row_tot_combine(const RowTot& a, const RowTot& b) {
    RowTot r;
    r.m = fmaxf(a.m, b.m);
    r.k = fmaxf(a.k, b.k);
    const double za = a.k == -INFINITY ? 0.0 : ldexp(a.z, (int)fmaxf(8.f * (a.k - r.k), -4096.f));
    const double zb = b.k == -INFINITY ? 0.0 : ldexp(b.z, (int)fmaxf(8.f * (b.k - r.k), -4096.f));
    r.z = za + zb;
    r.c = a.c + b.c;
    return r;
}
__device__ __forceinline__ double z_to_ref(double z, float k, float kr) {
    return k == -INFINITY ? 0.0 : ldexp(z, (int)fmaxf(8.f * (k - kr), -4096.f));
}
__device__ __forceinline__ RowTot rb_row_totals(RowTot t, RowShared& S) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const float wm = wave_max(t.m);
    const float wk = wave_max(t.k);
    const double wz = wave_sum(z_to_ref(t.z, t.k, wk));
    if (lane == 0) {
        S.tot_m[wave] = wm;
        S.tot_k[wave] = wk;
        S.tot_z[wave] = wz;
        S.tot_c[wave] = t.c;
    }
    __syncthreads();
    RowTot r{S.tot_m[0], S.tot_k[0], 0.0, S.tot_c[0]};
#pragma unroll
    for (int w = 1; w < kRW; ++w) {
        r.m = fmaxf(r.m, S.tot_m[w]);
        r.k = fmaxf(r.k, S.tot_k[w]);
        r.c += S.tot_c[w];
    }
    double zs[kRW];
#pragma unroll
    for (int w = 0; w < kRW; ++w) zs[w] = z_to_ref(S.tot_z[w], S.tot_k[w], r.k);
    static_assert(kRW == 8, "the cross-wave sum is written for eight waves");
    r.z = ((zs[0] + zs[1]) + (zs[2] + zs[3])) + ((zs[4] + zs[5]) + (zs[6] + zs[7]));
    return r;
}

// First capture threshold, from tile 0: about the rank-th largest thread
// maximum (binned over the range of thread maxima), so that at least `rank`
// logits of tile 0 are captured.
__device__ __forceinline__ float first_threshold(RowShared& S, float tm, int rank) {
    const float M0 = rb_max(tm, S.red_f);
    const bool fin = tm != -INFINITY;
    const float mn = rb_min(fin ? tm : INFINITY, S.red_f);
    const float span = M0 - mn;
    const float bscale = span > 0.f ? (float)(kNB - 1) / span : 0.f;
    for (int i = threadIdx.x; i < kNB; i += kRB) S.th_hc[i] = 0u;
    __syncthreads();
    const int b = fin ? min(kNB - 1, (int)((M0 - tm) * bscale)) : kNB;
    if (fin) atomicAdd(&S.th_hc[b], 1u);
    __syncthreads();
    if (threadIdx.x < 64) {
        int bin;
        u64 before, unused;
        wave_first_reach([&](int i) { return (u64)S.th_hc[i]; }, [](int) { return 0ull; }, (u64)rank, bin,
                         before, unused);
        if (threadIdx.x == 0) S.ibin = bin;
    }
    __syncthreads();
    const int b0 = S.ibin;
    // fewer finite thread maxima than `rank`: capture everything
    const float tau = b0 < 0 ? -INFINITY : rb_min((fin && b <= b0) ? tm : INFINITY, S.red_f);
    return tau;
}

// Weight 2^(x c - 8 kref) of a candidate in fp64 (kref: the row's
// power-of-two reference, so the weight is at most 1 up to the rounding of
// kref): the exponent is one fp64 FMA and exp2 is the fp64 routine, so the
// weight carries about one fp64 rounding.  Its fixed-point form (times 2^fx,
// truncated) drives the top-k / top-p decisions, whose sums must be exact and
// independent of order; the fp64 form gives the kept mass.
__device__ __forceinline__ double cand_weight(float x, float kref, double c) {
    return exp2(fmax(fma((double)x, c, -8.0 * (double)kref), -2000.0));
}
__device__ __forceinline__ u64 fixed_weight(double w, int fx) { return (u64)ldexp(w, fx); }

// Resolve top-k / top-p from the candidates.  Entries (up to kOwn per thread:
// its wave's candidates lane + 64 i) hold every logit >= the capture threshold.
// Masses are in units of 2^(8 kref) / scale (Zg: the row sum in units of
// 2^(8 kref)); z_kept is returned in units of 2^(8 kref).  Returns false when the candidates
// cannot decide (the caller then re-reads the row).  `side` runs once on
// wave 1 while wave 0 scans the bins, ahead of a barrier.
//
// The candidates are binned by value (kNB bins over [lo, M]) with their
// count and fixed-point mass.  Wave 0 scans the bins for the crossing bin
// and hands it to the others through LDS (the scan is VALU work that eight
// waves, two to a SIMD, would repeat for nothing); inside that bin the
// entries are gathered and every entry learns the count and mass of the
// bin's entries with a strictly larger key (wave 0 alone when the bin holds
// at most 64).  The bins and the gather counters were cleared when the row
// started.
template <int DT, class Side>
__device__ __forceinline__ bool resolve_reservoir(const RowArgs& a, RowShared& S, float M, float kref, double Zg,
                                                  int n_own, float tau, double scale, uint32_t& thr_key,
                                                  double& z_kept, int& n_kept, Side&& side) {
    const int tid = threadIdx.x, lane = tid & 63;
    const u64* mine = S.cand + (tid >> 6) * kCW + lane;  // this thread's candidates: mine[64 i], i < n_own
    uint32_t key[kOwn];
    u64 wt[kOwn];
    double ew[kOwn];  // fp64 weights (0 for unused slots)
    int bin[kOwn];
    float xmin = INFINITY;
    // every slot is read (those past n_own hold stale entries of the region
    // and are not used), so the reads need no branches and go out together
    u64 ent[kOwn];
#pragma unroll
    for (int i = 0; i < kOwn; ++i) ent[i] = mine[64 * i];
    // Straight-line over all slots (unused ones on a stand-in value), so the
    // slots' weight computations overlap.
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
        const bool use = i < n_own;
        const float x = use ? __uint_as_float((uint32_t)(ent[i] >> 32)) : M;
        key[i] = use ? fkey(x) : 0u;
        ew[i] = use ? cand_weight(x, kref, a.c64) : 0.0;
        wt[i] = fixed_weight(ew[i], a.fx_shift);
        xmin = use ? fminf(xmin, x) : xmin;
    }
    // every candidate is >= tau; a row captured whole has tau = -inf
    const float lo = tau != -INFINITY ? tau : rb_min(xmin, S.red_f);
    const float span = M - lo;
    const float bscale = span > 0.f ? (float)(kNB - 1) / span : 0.f;
#pragma unroll
    for (int i = 0; i < kOwn; ++i)
        bin[i] = i < n_own ? min(kNB - 1, (int)((M - key_to_float(key[i])) * bscale)) : kNB;
#pragma unroll
    for (int i = 0; i < kOwn; ++i) {
        if (i < n_own) {
            atomicAdd(&S.hc[bin[i]], 1u);
            atomicAdd(&S.hm[bin[i]], wt[i]);
        }
    }
    __syncthreads();

    // A bin of a bf16 row whose value range (widened by a quarter bin, far
    // beyond the rounding of the bin arithmetic) holds one bf16 value at or
    // above floor_key holds one key: its entries all tie.  bf16 keys are
    // t << 16 | (t >= 0x8000 ? 0 : 0xFFFF), increasing in t.
    auto single_key = [&](int b, uint32_t floor_key, uint32_t& kk) -> bool {
        if (DT != DT_BF16 || b >= kNB - 1 || !(bscale > 0.f)) return false;
        const float w = 1.f / bscale;
        if (!(w > 0x1p-16f * fabsf(M))) return false;
        auto k16 = [](uint32_t t) { return (t << 16) | (t >= 0x8000u ? 0u : 0xFFFFu); };
        const uint32_t klo = max(fkey(M - ((float)b + 1.25f) * w), floor_key);
        const uint32_t khi = b == 0 ? 0xFFFFFFFFu : fkey(M - ((float)b - 0.25f) * w);
        uint32_t tl = klo >> 16, th = khi >> 16;
        if (k16(tl) < klo) ++tl;
        if (k16(th) > khi) {
            if (th == 0u) return false;
            --th;
        }
        if (tl != th) return false;
        kk = k16(tl);
        return true;
    };
    // Exact decision inside bin b (entries with key >= floor_key, bcnt of
    // them with mass bmass): kept <=> base + (count or mass of the bin's
    // entries with a larger key) < limit.  The bin is the first to reach the
    // limit, so base < limit: tied entries are all kept.  Returns the
    // smallest kept key, the kept count and mass.
    auto resolve_bin = [&](int b, int call, uint32_t floor_key, u64 base, bool by_count, u64 limit, uint32_t bcnt,
                           u64 bmass, uint32_t& kmin, uint32_t& kcnt, u64& kmass) -> bool {
        {
            uint32_t kk;
            if (single_key(b, floor_key, kk)) {
                kmin = kk;
                kcnt = bcnt;
                kmass = bmass;
                return true;
            }
        }
        // gather (contention only among the bin's own entries)
        u64* bw = call == 0 ? S.bw : S.bw + kBinMax / 2;
        uint32_t* bk = call == 0 ? S.bkey : S.bkey + kBinMax / 2;
        constexpr int cap = kBinMax / 2;
#pragma unroll
        for (int i = 0; i < kOwn; ++i) {
            if (bin[i] == b && key[i] >= floor_key) {
                const int slot = atomicAdd(&S.nbin2[call], 1);
                if (slot < cap) {
                    bk[slot] = key[i];
                    bw[slot] = wt[i];
                }
            }
        }
        __syncthreads();
        const int nb = S.nbin2[call];
        if (nb > cap) return false;
        if (nb <= 64) {
            // one entry per lane of wave 0, which hands the result on
            if (tid < 64) {
                const uint32_t k = lane < nb ? bk[lane] : 0u;
                const u64 w = lane < nb ? bw[lane] : 0ull;
                uint32_t cgt = 0u;
                u64 mgt = 0ull;
                for (int jj = 0; jj < nb; ++jj) {
                    const uint32_t kj = lane_read(k, jj);
                    const u64 wj = lane_read(w, jj);
                    cgt += kj > k ? 1u : 0u;
                    mgt += kj > k ? wj : 0ull;
                }
                const bool kept = lane < nb && (by_count ? base + cgt < limit : base + mgt < limit);
                const uint32_t c = (uint32_t)__popcll(__ballot(kept));
                const u64 m = wave_allreduce(kept ? w : 0ull, [](u64 x, u64 y) { return x + y; });
                const uint32_t mn =
                    wave_allreduce(kept ? k : 0xFFFFFFFFu, [](uint32_t x, uint32_t y) { return x < y ? x : y; });
                if (tid == 0) {
                    S.bc_m = m;
                    S.bc_k[0] = c;
                    S.bc_k[1] = mn;
                }
            }
            __syncthreads();
            // (the next write to these slots follows the barriers of the next
            // crossing-bin search)
            kmass = S.bc_m;
            kcnt = S.bc_k[0];
            kmin = S.bc_k[1];
            return true;
        }
        uint32_t my_c = 0u;
        u64 my_m = 0ull;
        uint32_t my_min = 0xFFFFFFFFu;
        for (int i = tid; i < nb; i += kRB) {
            const uint32_t ki = bk[i];
            uint32_t cgt = 0u;
            u64 mgt = 0ull;
            for (int jj = 0; jj < nb; ++jj) {
                const uint32_t kj = bk[jj];
                if (kj > ki) {
                    ++cgt;
                    mgt += bw[jj];
                }
            }
            const bool kept = by_count ? (base + cgt < limit) : (base + mgt < limit);
            if (kept) {
                ++my_c;
                my_m += bw[i];
                my_min = min(my_min, ki);
            }
        }
        rb_count_mass_min(my_c, my_m, my_min, S);
        kcnt = my_c;
        kmass = my_m;
        kmin = my_min;
        return true;
    };

    // top-k: the bin holding the top_k-th largest logit, then exact ranks in it
    int bk = kNB;
    uint32_t tau_k = 0u, in_k_cnt = 0u;
    u64 in_k_mass = 0ull;
    u64 cb_k = 0ull, mb_k = 0ull;
    // wave 0 finds the crossing bin; the others take it from LDS (wave 1
    // runs `side` meanwhile, once)
    bool side_done = false;
    auto find_bcast = [&](auto&& va, auto&& vb, u64 target, int& b, u64& before_a, u64& before_b) {
        if (!side_done && (tid >> 6) == 1) side();
        side_done = true;
        if (tid < 64) {
            wave_first_reach(va, vb, target, b, before_a, before_b);
            if (tid == 0) {
                S.bc_i = b;
                S.bc_u[0] = before_a;
                S.bc_u[1] = before_b;
            }
        }
        __syncthreads();
        // (the next write to these slots follows a barrier of resolve_bin)
        b = S.bc_i;
        before_a = S.bc_u[0];
        before_b = S.bc_u[1];
    };
    if (a.use_k) {
        find_bcast([&](int i) { return (u64)S.hc[i]; }, [&](int i) { return S.hm[i]; }, (u64)a.top_k, bk, cb_k,
                   mb_k);
        if (bk < 0) return false;  // fewer than top_k entries captured
        if (!resolve_bin(bk, 0, 0u, cb_k, true, (u64)a.top_k, S.hc[bk], S.hm[bk], tau_k, in_k_cnt, in_k_mass))
            return false;
    }
    // The kept mass in fp64 (the fixed-point sums decide membership only):
    // each thread adds its kept candidates' weights in slot order, then the
    // block in a fixed order.
    auto kept_mass = [&](uint32_t tk) {
        double z = 0.0;
#pragma unroll
        for (int i = 0; i < kOwn; ++i) z += (i < n_own && key[i] >= tk) ? ew[i] : 0.0;
        return rb_sum(z, S.red_d);
    };
    const u64 zk = a.use_k ? mb_k + in_k_mass : 0ull;
    if (!a.use_p) {
        thr_key = tau_k;
        n_kept = (int)(cb_k + in_k_cnt);
        z_kept = kept_mass(tau_k);
        return true;
    }
    // top-p on the (top-k) kept set: kept <=> excl < ceil(top_p * Z * 2^s)
    const double zbase = a.use_k ? (double)zk / scale : Zg;
    u64 target = (u64)ceil((double)a.top_p * zbase * scale);
    if (target == 0ull) target = 1ull;
    if (a.use_k && target > zk) target = zk;  // rounding: keep the whole top-k set
    int bp;
    u64 mb_p, cb_p;
    find_bcast([&](int i) -> u64 { return i < bk ? S.hm[i] : (i == bk ? in_k_mass : 0ull); },
               [&](int i) -> u64 { return i < bk ? S.hc[i] : (i == bk ? in_k_cnt : 0u); }, target, bp, mb_p,
               cb_p);
    if (bp < 0) return false;  // the crossing lies below the candidates
    uint32_t kmin, kcnt;
    u64 kmass;
    if (!resolve_bin(bp, 1, bp == bk ? tau_k : 0u, mb_p, false, target, bp == bk ? in_k_cnt : S.hc[bp],
                     bp == bk ? in_k_mass : S.hm[bp], kmin, kcnt, kmass))
        return false;
    thr_key = kmin;
    n_kept = (int)(cb_p + kcnt);
    z_kept = kept_mass(kmin);
    return true;
}

// f(index, logit) over every logit of the row, each thread taking groups
// tid, tid + kRB, ... with kFE groups' loads in flight at once (indices past
// the row re-read its last group and are not passed on).
constexpr int kFE = 8;
template <int DT, class F>
__device__ __forceinline__ void row_for_each(const char* rowp, int V, F&& f) {
    constexpr int esz = DT == DT_BF16 ? 2 : 4;
    constexpr int per = 16 / esz;
    if ((((uintptr_t)rowp) & 15) == 0) {
        const int ng = V / per;
        for (int g0 = threadIdx.x; g0 < ng; g0 += kRB * kFE) {
            u32x4 raw[kFE];
#pragma unroll
            for (int u = 0; u < kFE; ++u) raw[u] = ld16_nt(rowp + (size_t)min(g0 + u * kRB, ng - 1) * 16);
#pragma unroll
            for (int u = 0; u < kFE; ++u) {
                const int g = g0 + u * kRB;
                if (g < ng) {
                    const uint32_t w[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
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
            }
        }
        for (int i = ng * per + threadIdx.x; i < V; i += kRB) f(i, load_logit(rowp, DT, i));
    } else {
        for (int i = threadIdx.x; i < V; i += kRB) f(i, load_logit(rowp, DT, i));
    }
}

constexpr int kGather = 4096;             // entries of one bin gathered into LDS by the re-read selection

// Exact selection by re-reading the row, for rows whose kept set the
// candidates cannot decide.  Over the keys >= floor_key: by_count, the
// largest key K whose count of keys >= K reaches `target` (the top-k value);
// otherwise the largest K whose fixed-point mass of keys >= K reaches
// `target` (the top-p crossing group).  Returns K with the count and mass of
// the keys above it and of its group.  Masses are grid weights (units of
// 2^(8 kref - fx)), as on the candidate path.
//
// Pass 1 bins the row by value: kNB bins from M down over 64 binary orders
// of magnitude of weight (lower values share the last bin), counts and
// masses in per-wave LDS histograms (no cross-wave contention) merged in
// wave order.  Masses are taken relative to each bin's top (see below), so
// a logit costs one fp32 exp2.  Inside the bin where the target is reached, an 8-bit radix
// over the keys, below the prefix that every key of the bin shares, finds the
// exact group.  The bin's entries are gathered into LDS in one more pass
// when they fit (kGather), and counted per digit there; otherwise the row is
// re-read for every digit, with atomics only for that bin's entries.
template <int DT>
__device__ __forceinline__ Sel row_select_reread(RowShared& S, const RowArgs& a, const char* rowp, int V, float M, float kref,
                                 uint32_t floor_key, bool by_count, u64 target) {
    const int tid = threadIdx.x, wave = tid >> 6;
    static_assert(sizeof(u64) * kRW * kNB <= sizeof(S.u) && sizeof(uint32_t) * kRW * kNB <= sizeof(S.cand),
                  "per-wave histograms fit the reservoir space");
    static_assert(sizeof(u64) * kGather <= sizeof(S.u) && sizeof(uint32_t) * kGather <= sizeof(S.cand),
                  "a gathered bin fits the reservoir space");
    u64* pm = reinterpret_cast<u64*>(&S.u);             // [kRW][kNB] masses
    uint32_t* pc = reinterpret_cast<uint32_t*>(S.cand);  // [kRW][kNB] counts
    const float span = (float)(64.0 / a.c64);            // logit range of 64 binary orders of weight
    const float bscale = (float)(kNB - 1) / span;
    auto vbin = [&](float x) { return (int)fminf((M - x) * bscale, (float)(kNB - 1)); };
    // Weights relative to the top of each value bin: w = G_b * 2^((x - x_b) c)
    // with the factor 2^((x - x_b) c) in [2^-1/8, 1] taken in fp32 (a small
    // exponent, so about one ulp) and held in 31-bit fixed point; G_b, the
    // bin's scale into the row's fixed-point units, applies once per bin.
    const float cf = (float)a.c64;
    auto xtop = [&](int b) { return M - (float)b / bscale; };
    auto local_w = [&](float x, int b) -> u64 {
        const float e = fminf((x - xtop(b)) * cf, 0.f);
        return (u64)(uint32_t)(__builtin_amdgcn_exp2f(e) * 2147483648.0f);
    };
    auto bin_scale = [&](int b) {
        return exp2((double)xtop(b) * a.c64 - 8.0 * (double)kref + (double)(a.fx_shift - 31));
    };

    __syncthreads();  // the reservoir space is free
    for (int i = tid; i < kRW * kNB; i += kRB) {
        pm[i] = 0ull;
        pc[i] = 0u;
    }
    __syncthreads();
    u64* my_m = pm + wave * kNB;
    uint32_t* my_c = pc + wave * kNB;
    row_for_each<DT>(rowp, V, [&](int, float x) {
        if (fkey(x) >= floor_key) {
            const int b = vbin(x);
            atomicAdd(&my_m[b], local_w(x, b));
            atomicAdd(&my_c[b], 1u);
        }
    });
    __syncthreads();
    for (int b = tid; b < kNB; b += kRB) {
        u64 m = 0ull;
        uint32_t c = 0u;
#pragma unroll
        for (int w = 0; w < kRW; ++w) {
            m += pm[w * kNB + b];
            c += pc[w * kNB + b];
        }
        S.hm[b] = (u64)((double)m * bin_scale(b));
        S.hc[b] = c;
    }
    __syncthreads();
    Sel r;
    r.ok = 0;
    r.key = 0u;
    r.above = r.group = 0ull;
    r.cnt_above = r.cnt_group = 0u;
    // every wave finds the bin where the target is reached (same data, same result)
    int bin;
    u64 bsel, both;
    if (by_count)
        wave_first_reach([&](int i) { return (u64)S.hc[i]; }, [&](int i) { return S.hm[i]; }, target, bin, bsel,
                         both);
    else
        wave_first_reach([&](int i) { return S.hm[i]; }, [&](int i) { return (u64)S.hc[i]; }, target, bin, bsel,
                         both);
    if (bin < 0) return r;  // the totals stay below the target
    u64 A = by_count ? both : bsel;                   // mass above the bin
    uint32_t C = (uint32_t)(by_count ? bsel : both);  // count above
    const double G = bin_scale(bin);
    u64 A_in = 0ull;  // mass above inside the bin, bin-local units
    // keys every entry of the bin lies between (its value bounds, widened by
    // a fraction of a bin against rounding in vbin)
    const float v_hi = bin == 0 ? INFINITY : M - ((float)bin - 0.0625f) / bscale;
    const float v_lo = bin == kNB - 1 ? -INFINITY : M - ((float)bin + 1.0625f) / bscale;
    const uint32_t k_lo = max(fkey(v_lo), floor_key), k_hi = fkey(v_hi);
    const uint32_t diff = k_lo ^ k_hi;
    if (diff == 0u) {  // one key only
        r.ok = 1;
        r.key = k_lo;
        r.above = A;
        r.cnt_above = C;
        r.group = S.hm[bin];
        r.cnt_group = S.hc[bin];
        return r;
    }
    const int top_bit = 31 - __clz((int)diff);
    uint32_t mask = top_bit >= 24 ? 0u : (0xFFFFFFFFu << (((top_bit >> 3) + 1) * 8));
    uint32_t prefix = k_lo & mask;
    // A bin that fits is gathered into LDS once (keys and weights), and its
    // digits are counted there; a larger one is re-read for every digit.
    const int nb = (int)S.hc[bin];
    const bool gathered = nb <= kGather;
    uint32_t* gkey = pc;  // the histograms are merged: their space is free
    u64* gw = pm;
    if (gathered) {
        if (tid == 0) S.nlist = 0;
        __syncthreads();
        row_for_each<DT>(rowp, V, [&](int, float x) {
            const uint32_t k = fkey(x);
            const bool hit = k >= floor_key && vbin(x) == bin;
            const u64 m = __builtin_amdgcn_ballot_w64(hit);
            if (m) {  // one atomic per wave and call
                const int leader = __ffsll((long long)m) - 1;
                int base = 0;
                if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(&S.nlist, __popcll(m));
                base = __builtin_amdgcn_readlane(base, leader);
                const int slot = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                      __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                if (hit && slot < kGather) {
                    gkey[slot] = k;
                    gw[slot] = local_w(x, bin);
                }
            }
        });
        __syncthreads();
    }
    for (int shift = (top_bit >> 3) * 8; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += kRB) {
            S.bw[i] = 0ull;
            S.bkey[i] = 0u;
        }
        __syncthreads();
        auto count_digit = [&](uint32_t k, u64 w) {
            if ((k & mask) == prefix) {
                const uint32_t d = (k >> shift) & 255u;
                atomicAdd(&S.bw[d], w);
                atomicAdd(&S.bkey[d], 1u);
            }
        };
        if (gathered) {
            for (int e = tid; e < nb; e += kRB) count_digit(gkey[e], gw[e]);
        } else {
            row_for_each<DT>(rowp, V, [&](int, float x) {
                const uint32_t k = fkey(x);
                if (k >= floor_key && vbin(x) == bin) count_digit(k, local_w(x, bin));
            });
        }
        __syncthreads();
        // digits from the top: index i is digit 255 - i
        int di;
        u64 dsel, doth;
        // what is still needed, in count or in bin-local mass
        const u64 rest = by_count ? (u64)(target - C)
                                  : max(1ull, (u64)ceil((double)(target - A) / G) - A_in);
        if (by_count)
            wave_first_reach([&](int i) { return i < 256 ? (u64)S.bkey[255 - i] : 0ull; },
                             [&](int i) { return i < 256 ? S.bw[255 - i] : 0ull; }, rest, di, dsel, doth);
        else
            wave_first_reach([&](int i) { return i < 256 ? S.bw[255 - i] : 0ull; },
                             [&](int i) { return i < 256 ? (u64)S.bkey[255 - i] : 0ull; }, rest, di, dsel, doth);
        if (di < 0) return r;  // cannot happen with consistent passes; the caller keeps the whole range
        const uint32_t d = 255u - (uint32_t)di;
        A_in += by_count ? doth : dsel;
        C += (uint32_t)(by_count ? dsel : doth);
        prefix |= d << shift;
        mask |= 0xFFu << shift;
        if (shift == 0) {
            r.group = (u64)((double)S.bw[d] * G);
            r.cnt_group = S.bkey[d];
        }
        __syncthreads();  // every wave has read the digit histogram
    }
    r.ok = 1;
    r.key = prefix;
    r.above = A + (u64)((double)A_in * G);
    r.cnt_above = C;
    return r;
}

// One row.  MODE_PLAIN / MODE_NUCLEUS keep, per thread, the sum of
// 2^(x * log2(e) / T - 8 k) over the thread's logits, where the reference
// 8 k is the smallest multiple of 8 at or above the thread's largest
// x * log2(e) / T so far: every term is at most 1, a change of reference is
// an exact power-of-two rescale (ldexp), and -8 k is an exact float.  The
// exponent is one FMA, x * c_hi - 8 k, with c_hi = c - c_lo the largest
// float below c = log2(e) / T: the sum is of 2^(x c_hi - 8 k).  Against the
// row maximum M that is Z = sum 2^((x - M) c_hi), within c_lo ln2 E[M - x]
// (under the softmax weights, a few binary orders times c 2^-23) of the sum
// with c itself; sums in units of 2^(8 kref) of the exact c take the factor
// 2^(M c_lo).
template <int DT, int MODE>
__device__ __forceinline__ void row_body(const RowArgs& a, RowShared& S, int row) {
    const char* rowp = row_ptr(a.sh, row);
    const int V = a.sh.V;
    constexpr bool kFilt = MODE != MODE_PLAIN;
    constexpr bool kSum = MODE != MODE_TOPK;
    const RowStream<DT> st(rowp, V);
    constexpr int NL = RowStream<DT>::NL;
    constexpr int per = RowStream<DT>::per;

    // Streaming waves issue ahead of waves of a co-resident workgroup that
    // are already finishing their row (priority drops again below).
    __builtin_amdgcn_s_setprio(1);
    // the drafted token's logit, fetched while the row streams
    // (thread 0 writes the record; thread 64 takes the token's weight off
    // the path of wave 0 during the resolution)
    int d_tok = -1;
    float xd = -INFINITY;
    if ((threadIdx.x == 0 || threadIdx.x == 64) && row_has_token(a.sh, row)) {
        d_tok = row_token(a.sh, row);
        if (d_tok >= 0 && d_tok < V) xd = load_logit(rowp, DT, d_tok);
    }
    float m_th = -INFINITY;  // running maximum of this thread's logits
    float k_th = -INFINITY;  // reference index k (a whole number, as a float)
    double z_th = 0.0;       // sum of 2^(x * log2(e) / T - 8 k_th) over this thread's logits
    float tau = INFINITY;    // capture threshold of this wave
    float tau0 = INFINITY;   // the first (block-wide) threshold: at or below every wave's
    float m_run = -INFINITY; // running maximum for threshold refreshes (top-k rows)
    int fill = 0, ovf = 0;   // this wave's segment (uniform per wave)
    if (kFilt) {
        // bins of the candidate resolution (first used after many barriers)
        for (int i = threadIdx.x; i < kNB; i += kRB) {
            S.hm[i] = 0ull;
            S.hc[i] = 0u;
        }
        if (threadIdx.x < 2) S.nbin2[threadIdx.x] = 0;
    }

    // One tile of kREPT logits per thread (NL groups of `per`; group j of this
    // thread is gbase + j * gstride): group maxima, running max and sum,
    // capture.  The first tile also sets the capture threshold: the kR0-th
    // (nucleus) or top_k-th (top-k) largest thread maximum of the block, so
    // at least that many logits are captured.
    auto core = [&](const float (&v)[kREPT], const u32x4 (&unit)[NL], int gbase, int gstride, bool first) {
        float gm[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            float g = v[j * per];
#pragma unroll
            for (int q = 1; q < per; ++q) g = fmaxf(g, v[j * per + q]);
            gm[j] = g;
        }
        float tm = gm[0];
#pragma unroll
        for (int j = 1; j < NL; ++j) tm = fmaxf(tm, gm[j]);
        if (kSum) {
            m_th = fmaxf(m_th, tm);
            // k of this tile: ceil(tm * log2(e) / (8 T)); a float rounding
            // that lands one short only lets terms exceed 1 by a hair
            const float kt = ceilf(tm * a.c8);
            if (kt > k_th) {
                // new reference: rescale by 2^(8 (k_th - kt)), exact (z_th is
                // still 0 while no finite logit has been seen)
                z_th = k_th == -INFINITY ? 0.0 : ldexp(z_th, (int)fmaxf(8.f * (k_th - kt), -4096.f));
                k_th = kt;
            }
            if (k_th != -INFINITY) {
                const float nmc = -8.f * k_th;
                // four partial sums, each started by its first term
                float acc[4];
#pragma unroll
                for (int s = 0; s < kREPT; ++s) {
                    const float e = fmaf(v[s], a.c_hi, nmc);
                    const float term = __builtin_amdgcn_exp2f(e);
                    acc[s & 3] = s < 4 ? term : acc[s & 3] + term;
                }
                z_th += (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
            }
        }
        if (kFilt) {
            if (MODE == MODE_TOPK) m_run = fmaxf(m_run, tm);
            if (first) {
                tau = V <= kCW ? -INFINITY
                                : first_threshold(S, tm, MODE == MODE_TOPK ? max(1, min(a.top_k, kRB)) : kR0);
                tau0 = tau;
            }
            capture_units<NL>(S, unit, gm, gbase, gstride, tau, fill, ovf);
        }
    };

    // Top-k rows raise the threshold after tiles 3 and 15 from the running
    // thread maxima: any value with top_k logits at or above it bounds the
    // row's top_k-th largest from below; it only rises, so every logit at or
    // above the final threshold is held.
    auto refresh = [&](int t) {
        if (MODE == MODE_TOPK && (t == 3 || t == 15)) {
            tau = fmaxf(tau, first_threshold(S, m_run, max(1, min(a.top_k, kRB))));
        }
    };
    // The captured units are expanded into the wave's candidates 64 at a
    // time while the row streams, so that a wave has few of them left to
    // expand when its stream ends.
    int n_w = 0;   // this wave's candidates (uniform per wave)
    int done = 0;  // units of the segment expanded so far (uniform per wave)
    auto expand_batch = [&]() {
        if (kFilt && fill - done >= 64) {
            const u64 w = wave_expand<DT>(S, V, tau, done, fill, ovf, n_w);
            n_w = (int)(uint32_t)w;
            ovf = (int)(w >> 32);
            done += 64;
        }
    };
    auto expand_rest = [&]() {
        if (kFilt) {
            for (; done < fill; done += 64) {
                const u64 w = wave_expand<DT>(S, V, tau, done, fill, ovf, n_w);
                n_w = (int)(uint32_t)w;
                ovf = (int)(w >> 32);
            }
        }
    };
    auto full_tile = [&](int t, const u32x4 (&raw)[NL]) {
        float v[kREPT];
        RowStream<DT>::unpack_full(raw, v);
        core(v, raw, t * (kRB * NL) + (int)threadIdx.x, kRB, t == 0);
        refresh(t);
        expand_batch();
    };
    auto any_tile = [&](int t, const u32x4 (&raw)[NL]) {
        float v[kREPT];
        st.unpack(t, raw, v);
        u32x4 unit[NL];
#pragma unroll
        for (int j = 0; j < NL; ++j) unit[j] = RowStream<DT>::repack(v, j);
        core(v, unit, t * (kRB * NL) + (int)threadIdx.x, kRB, t == 0);
        refresh(t);
    };
    {
        // Steady state: NS = 4 full tiles of loads in flight in rotating
        // registers, straight-line code so that each tile waits only for its
        // own loads (eight for bf16 rows, the same registers, was slower).
        // Rows with fewer than five full tiles go tile by tile.
        const int nf = st.nfull;
        int t = 0;
        auto rotate = [&](auto ns) {
            constexpr int NS = decltype(ns)::value;
            u32x4 rs[NS][NL];
#pragma unroll
            for (int q = 0; q < NS; ++q) st.issue_full(q, rs[q]);
            full_tile(0, rs[0]);
            st.issue_full(NS, rs[0]);
            t = 1;
            // Every scalar load is complete here (lgkmcnt(0), other counters
            // left alone): without it the compiler waits on lgkmcnt inside the
            // loop, and with capture stores in flight that wait is for the LDS.
            __builtin_amdgcn_s_waitcnt(0xC07F);
            for (; t + 2 * NS - 1 < nf; t += NS) {
#pragma unroll
                for (int q = 0; q < NS; ++q) {
                    full_tile(t + q, rs[(1 + q) % NS]);
                    st.issue_full(t + q + NS, rs[(1 + q) % NS]);
                }
            }
            // drain: the rest of the row (at most NS more tiles, the last
            // possibly partial) rides the same rotation with clamped loads
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                full_tile(t + q, rs[(1 + q) % NS]);
                st.issue_clamped(t + q + NS, rs[(1 + q) % NS]);
            }
            t += NS;
#pragma unroll
            for (int q = 0; q < NS; ++q)
                if (t + q < st.nt) any_tile(t + q, rs[(1 + q) % NS]);
            t = st.nt;
        };
        if (nf >= 5) rotate(std::integral_constant<int, 4>());
        u32x4 rA[NL];
        for (; t < st.nt; ++t) {
            st.issue(t, rA);
            any_tile(t, rA);
        }
    }

    __builtin_amdgcn_s_setprio(0);
    // ---- merge the row (fixed-order reductions) ----
    int n_own = 0;
    u64 cflags = 0ull;
    if (kFilt) {
        expand_rest();
        n_own = min(kOwn, max(0, (n_w - (int)(threadIdx.x & 63) + 63) / 64));
        // one contribution per wave: count | overflow << 32
        cflags = (u64)n_w | ((u64)(ovf ? 1 : 0) << 32);
    }
    // the barrier of the block totals also ends every wave's use of its segment
    const RowTot tot =
        rb_row_totals(RowTot{MODE == MODE_TOPK ? m_run : m_th, kSum ? k_th : -INFINITY, z_th, cflags}, S);
    const float M = tot.m;
    const int n_res = (tot.c >> 32) ? kCap + 1 : (int)(uint32_t)tot.c;

    float thr = -INFINITY;
    int n_kept = V;
    int flags = 0;
    double Z = 0.0;       // the row sum relative to the row maximum
    double z_kept = 0.0;  // the kept mass relative to the row maximum
    double ptok = 0.0;    // thread 0: the drafted token's probability, when it is kept

    if (!kFilt) {
        // z * 2^(8 k - M c_hi)
        Z = (kSum && tot.k != -INFINITY) ? tot.z * exp2(8.0 * (double)tot.k - (double)M * (double)a.c_hi) : 0.0;
        z_kept = Z;
        if (threadIdx.x == 0 && d_tok >= 0 && d_tok < V) ptok = exp(((double)xd - (double)M) * a.inv_T) / Z;
    } else {
        flags = SPEC_ROW_FILTERED;
        const double scale = ldexp(1.0, a.fx_shift);
        uint32_t thr_key = 0u;
        // power-of-two reference of the row: the streaming sums use the same
        // (a thread's reference is ceil(its max * c / 8))
        const float kref = M != -INFINITY ? ceilf(M * a.c8) : 0.f;
        // the row sum in grid units (2^(8 kref) of the exact c; one grid unit
        // is 2^(8 kref - M c) against the row maximum): the streamed sum of
        // 2^(x c_hi - 8 kref) times 2^(M c_lo) (a series, |M c_lo| being tiny)
        const double ml = (double)M * (double)a.c_lo * 0.6931471805599453;
        const double Zg = (kSum && tot.k != -INFINITY)
                              ? ldexp(tot.z, (int)(8.f * (tot.k - kref))) * (1.0 + ml * (1.0 + ml * (0.5 + ml / 6.0)))
                              : 0.0;
        // Wave 1 takes the grid unit and the drafted token's weight in grid
        // units (two fp64 exp2) while wave 0 searches the bins.
        auto side = [&]() {
            const double zs = exp2(8.0 * (double)kref - (double)M * a.c64);
            const double pt = exp2((double)xd * a.c64 - 8.0 * (double)kref);
            if (threadIdx.x == 64) {
                S.side_zs = zs;
                S.side_pt = pt;
            }
        };
        double zk_grid = 0.0;
        bool fast = n_res <= kCap &&
                    resolve_reservoir<DT>(a, S, M, kref, Zg, n_own, tau0, scale, thr_key, zk_grid, n_kept, side);
        if (fast) {
            thr = key_to_float(thr_key);
            const double zs = S.side_zs;
            z_kept = zk_grid * zs;
            Z = Zg * zs;
            if (threadIdx.x == 0) ptok = S.side_pt / zk_grid;
        } else {
            flags |= SPEC_ROW_EXACT_PATH;
            const double zs = exp2(8.0 * (double)kref - (double)M * a.c64);
            Z = Zg * zs;
            uint32_t thk = 0u;
            uint32_t cnt = (uint32_t)V;
            u64 zfx = 0ull;  // kept mass, grid units
            bool have_z = false;
            if (a.use_k) {
                const Sel sk = row_select_reread<DT>(S, a, rowp, V, M, kref, 0u, true, (u64)a.top_k);
                if (sk.ok) {
                    thk = sk.key;
                    cnt = sk.cnt_above + sk.cnt_group;
                    zfx = sk.above + sk.group;
                    have_z = true;
                }
            }
            if (a.use_p) {
                // top-p on the (top-k) kept set: the target mass in grid units
                const double zbase = have_z ? (double)zfx : Zg * scale;
                u64 target = (u64)ceil((double)a.top_p * zbase);
                if (target == 0ull) target = 1ull;
                if (have_z && target > zfx) target = zfx;  // rounding: keep the whole top-k set
                const Sel sp = row_select_reread<DT>(S, a, rowp, V, M, kref, thk, false, target);
                if (sp.ok) {
                    thk = sp.key;
                    zfx = sp.above + sp.group;
                    cnt = sp.cnt_above + sp.cnt_group;
                    have_z = true;
                }
            }
            // key 0 (no selection applied) keeps every logit
            thr = thk == 0u ? -INFINITY : key_to_float(thk);
            n_kept = (int)cnt;
            // The kept mass relative to the row maximum in fp64: one more pass
            // over the row, an fp64 exp for each kept logit (each thread adds
            // its own in a fixed order, then the block).
            double zt = 0.0;
            row_for_each<DT>(rowp, V, [&](int, float x) {
                if (fkey(x) >= thk) zt += exp(((double)x - (double)M) * a.inv_T);
            });
            z_kept = rb_sum(zt, S.red_d);
            if (threadIdx.x == 0 && d_tok >= 0 && d_tok < V)
                ptok = exp(((double)xd - (double)M) * a.inv_T) / z_kept;
        }
        // kept list of a target row, sorted by token index.  Fast path: every
        // wave's candidates are in index order (a wave captures its groups in
        // ascending order), so each wave packs its kept ones in place and an
        // entry's place in the merged list is its place in its own wave's
        // list plus, for every other wave, the number of that wave's kept
        // indices below it.  Exact path: gather the kept logits in a pass over
        // the row, bucket them by tile and rank each inside its bucket.  Both
        // orders are deterministic.
        if (row < a.sh.n_trows && a.want_list) {
            const int list_n = (n_kept <= kListMax && st.nt <= kNB) ? n_kept : -1;
            const uint32_t tk = fkey(thr);
            uint2* out = a.kept + (size_t)row * kListMax;
            // Each listed token also gets its probability p and, with a draft
            // row at this position, the draft's logit, read now (this row has
            // slack before the draft rows finish), so the draw needs neither
            // an exp for p nor a gather of its own.
            const int kpos_row = row % (a.sh.K + 1);
            const bool with_draft = a.sh.n_drows > 0 && kpos_row < seq_len(a.sh, row / (a.sh.K + 1));
            const char* dp = with_draft ? row_ptr(a.sh, a.sh.n_trows + (row / (a.sh.K + 1)) * a.sh.K + kpos_row)
                                        : nullptr;
            float* outd = a.kept_d + (size_t)row * kListMax;
            double* outp = a.kept_p + (size_t)row * kListMax;
            const double inv_zk = 1.0 / z_kept;
            auto emit = [&](int rank, uint32_t idx, uint32_t bits) {
                out[rank] = make_uint2(idx, bits);
                outp[rank] = exp(((double)__uint_as_float(bits) - (double)M) * a.inv_T) * inv_zk;
                if (with_draft) outd[rank] = load_logit(dp, a.sh.ddt, idx);
            };
            // Tokens come in blocks of 64 groups (64 * per tokens) that each
            // belong to one wave (block b to wave b mod kRW), and a wave's
            // list holds its blocks' entries contiguously in block order.  So
            // an entry's rank is the number of kept entries in all earlier
            // blocks plus its place within its block's run.
            constexpr int kBlkShift = DT == DT_BF16 ? 9 : 8;  // log2(64 * per)
            const int nblk = (V + (1 << kBlkShift) - 1) >> kBlkShift;
            if (list_n >= 0 && fast && nblk <= kNB) {
                const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
                u64* region = S.cand + wave * kCW;
                // per block: kept count (th_hc), then its exclusive prefix;
                // first list position of its run (hm)
                for (int i = threadIdx.x; i < nblk; i += kRB) {
                    S.th_hc[i] = 0u;
                    S.hm[i] = ~0ull;
                }
                u64 own[kOwn];
#pragma unroll
                for (int i = 0; i < kOwn; ++i) own[i] = i < n_own ? region[lane + 64 * i] : 0ull;
                __builtin_amdgcn_wave_barrier();
                int p = 0;
                int kpos[kOwn];  // list position of this lane's kept entries, or -1
#pragma unroll
                for (int i = 0; i < kOwn; ++i) {
                    const bool keep = i < n_own && fkey(__uint_as_float((uint32_t)(own[i] >> 32))) >= tk;
                    const u64 m = __builtin_amdgcn_ballot_w64(keep);
                    const int r = p + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    kpos[i] = keep ? r : -1;
                    p += __popcll(m);
                }
                __syncthreads();  // the bins are cleared
#pragma unroll
                for (int i = 0; i < kOwn; ++i) {
                    if (kpos[i] >= 0) {
                        const uint32_t blk = (uint32_t)own[i] >> kBlkShift;
                        atomicAdd(&S.th_hc[blk], 1u);
                        atomicMin(&S.hm[blk], (u64)kpos[i]);
                    }
                }
                __syncthreads();
                int nk_all = 0;
                const int cnt = (int)threadIdx.x < nblk ? (int)S.th_hc[threadIdx.x] : 0;
                const int before = rb_excl_scan(cnt, S.red_i, nk_all);
                if ((int)threadIdx.x < nblk) S.th_hc[threadIdx.x] = (uint32_t)before;
                __syncthreads();
                const int nk = min(nk_all, list_n);
#pragma unroll
                for (int i = 0; i < kOwn; ++i) {
                    if (kpos[i] >= 0) {
                        const uint32_t idx = (uint32_t)own[i];
                        const uint32_t blk = idx >> kBlkShift;
                        const int rank = (int)S.th_hc[blk] + kpos[i] - (int)S.hm[blk];
                        if (rank < nk) emit(rank, idx, (uint32_t)(own[i] >> 32));
                    }
                }
            } else if (list_n >= 0 && fast) {
                const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
                u64* region = S.cand + wave * kCW;
                u64 own[kOwn];
#pragma unroll
                for (int i = 0; i < kOwn; ++i) own[i] = i < n_own ? region[lane + 64 * i] : 0ull;
                __builtin_amdgcn_wave_barrier();
                int p = 0;
#pragma unroll
                for (int i = 0; i < kOwn; ++i) {
                    const bool keep = i < n_own && fkey(__uint_as_float((uint32_t)(own[i] >> 32))) >= tk;
                    const u64 m = __builtin_amdgcn_ballot_w64(keep);
                    const int r = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                 __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                    if (keep) region[p + r] = own[i];
                    p += __popcll(m);
                }
                if (lane == 0) S.red_i[wave] = p;
                __syncthreads();
                int kw[kRW], off[kRW];
                int nk = 0;
#pragma unroll
                for (int w = 0; w < kRW; ++w) {
                    kw[w] = S.red_i[w];
                    off[w] = nk;
                    nk += kw[w];
                }
                nk = min(nk, list_n);
                for (int e = threadIdx.x; e < nk; e += kRB) {
                    int w0 = 0;
#pragma unroll
                    for (int w = 1; w < kRW; ++w) w0 = e >= off[w] ? w : w0;
                    const u64 me = S.cand[w0 * kCW + (e - off[w0])];
                    const uint32_t idx = (uint32_t)me;
                    // kept indices below idx in every wave's list (its own
                    // included, where that is its position), by binary
                    // searches run side by side
                    const uint32_t* L = reinterpret_cast<const uint32_t*>(S.cand);
                    int lo[kRW];
#pragma unroll
                    for (int w = 0; w < kRW; ++w) lo[w] = 0;
                    static_assert(kCW <= 511, "the search covers lists of up to 511 entries");
#pragma unroll
                    for (int step = 256; step >= 1; step >>= 1) {
                        // all eight probes are read before any is used (one
                        // LDS round trip per step); a probe at the list's
                        // end repeats its last entry, which never moves lo
                        int probe[kRW];
                        uint32_t val[kRW];
#pragma unroll
                        for (int w = 0; w < kRW; ++w) {
                            probe[w] = min(lo[w] + step, kw[w]);
                            val[w] = L[2 * (w * kCW + max(probe[w], 1) - 1)];
                        }
#pragma unroll
                        for (int w = 0; w < kRW; ++w) lo[w] = (probe[w] > lo[w] && val[w] < idx) ? probe[w] : lo[w];
                    }
                    int rank = 0;
#pragma unroll
                    for (int w = 0; w < kRW; ++w) rank += lo[w];
                    if (rank < nk) emit(rank, idx, (uint32_t)(me >> 32));
                }
            } else if (list_n >= 0) {
                constexpr int kLPT = kListMax / kRB;
                u64 own[kLPT];
                __syncthreads();
                if (threadIdx.x == 0) S.nlist = 0;
                __syncthreads();
                row_for_each<DT>(rowp, V, [&](int i, float x) {
                    // one atomic per wave and call: the first hit lane reserves
                    // the wave's slots
                    const bool hit = x >= thr;
                    const u64 m = __builtin_amdgcn_ballot_w64(hit);
                    if (m) {
                        const int leader = __ffsll((long long)m) - 1;
                        int base = 0;
                        if ((int)(threadIdx.x & 63) == leader) base = atomicAdd(&S.nlist, __popcll(m));
                        base = __builtin_amdgcn_readlane(base, leader);
                        const int p = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                        if (hit && p < kListMax) S.u.list[p] = ((u64)__float_as_uint(x) << 32) | (uint32_t)i;
                    }
                });
                __syncthreads();
                const int nk = min(S.nlist, list_n);
                // bucket = streaming tile of the token
                for (int i = threadIdx.x; i < kNB; i += kRB) {
                    S.hc[i] = 0u;
                    S.bkey[i] = 0u;
                }
#pragma unroll
                for (int i = 0; i < kLPT; ++i) {
                    const int slot = threadIdx.x + i * kRB;
                    own[i] = slot < nk ? S.u.list[slot] : 0ull;
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < kLPT; ++i)
                    if (threadIdx.x + i * kRB < nk) atomicAdd(&S.hc[(uint32_t)own[i] / kRTile], 1u);
                __syncthreads();
                if (threadIdx.x < 64) {
                    // exclusive prefix of bucket counts, bucket starts into hm
                    constexpr int per = kNB / 64;
                    const int lane = threadIdx.x;
                    u64 c[per];
                    u64 ls = 0ull;
#pragma unroll
                    for (int q = 0; q < per; ++q) {
                        c[q] = S.hc[per * lane + q];
                        ls += c[q];
                    }
                    u64 run = wave_incl_scan(ls) - ls;
#pragma unroll
                    for (int q = 0; q < per; ++q) {
                        S.hm[per * lane + q] = run;
                        run += c[q];
                    }
                }
                __syncthreads();
#pragma unroll
                for (int i = 0; i < kLPT; ++i) {
                    if (threadIdx.x + i * kRB < nk) {
                        const uint32_t bkt = (uint32_t)own[i] / kRTile;
                        const uint32_t p = (uint32_t)S.hm[bkt] + atomicAdd(&S.bkey[bkt], 1u);
                        S.u.list[p] = own[i];
                    }
                }
                __syncthreads();
                for (int e = threadIdx.x; e < nk; e += kRB) {
                    const u64 me = S.u.list[e];
                    const uint32_t idx = (uint32_t)me;
                    const uint32_t bkt = idx / kRTile;
                    const int s0 = (int)S.hm[bkt], len = (int)S.hc[bkt];
                    int rank = 0;
                    for (int q = s0; q < s0 + len; ++q) rank += ((uint32_t)S.u.list[q] < idx) ? 1 : 0;
                    emit(s0 + rank, idx, (uint32_t)(me >> 32));
                }
            }
            if (threadIdx.x == 0) a.kept_n[row] = list_n;
        }
    }

    if (threadIdx.x == 0) {
        RowRec r;
        r.s.max_logit = M;
        r.z_all = kSum ? Z : __longlong_as_double(0x7FF8000000000000LL);  // NaN: not computed
        r.pad = 0.0;
        r.s.thresh = thr;
        r.s.n_kept = n_kept;
        r.s.flags = flags;
        r.s.z_kept = z_kept;
        double prob = __longlong_as_double(0x7FF8000000000000LL);  // NaN: no drafted token
        if (row_has_token(a.sh, row)) {
            prob = 0.0;
            if (d_tok >= 0 && d_tok < V && xd >= thr) prob = ptok;
        }
        r.s.prob_at_token = prob;
        a.rec[row] = r;
    }
}

// The record of a split unfiltered row from its parts, combined in part
// order (one thread; the parts' records were stored with agent-scope stores
// before their arrivals were counted).
__device__ __forceinline__ void merge_row(const RowArgs& a, int row) {
    RowTot t{-INFINITY, -INFINITY, 0.0, 0ull};
    for (int p = 0; p < a.parts; ++p) {
        const PartRec* q = a.prec + (size_t)row * a.parts + p;
        const float qm = __hip_atomic_load(&q->m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float qk = __hip_atomic_load(&q->k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const double qz = __hip_atomic_load(&q->z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        t = row_tot_combine(t, RowTot{qm, qk, qz, 0ull});
    }
    const float M = t.m;
    const double Z = t.k != -INFINITY ? t.z * exp2(8.0 * (double)t.k - (double)M * (double)a.c_hi) : 0.0;
    const int V = a.sh.V;
    RowRec r;
    r.s.max_logit = M;
    r.z_all = Z;
    r.pad = 0.0;
    r.s.thresh = -INFINITY;
    r.s.n_kept = V;
    r.s.flags = 0;
    r.s.z_kept = Z;
    double prob = __longlong_as_double(0x7FF8000000000000LL);  // NaN: no drafted token
    if (row_has_token(a.sh, row)) {
        prob = 0.0;
        const int d_tok = row_token(a.sh, row);
        if (d_tok >= 0 && d_tok < V) {
            const float xd = load_logit(row_ptr(a.sh, row), row_dt(a.sh, row), d_tok);
            prob = exp(((double)xd - (double)M) * a.inv_T) / Z;
        }
    }
    r.s.prob_at_token = prob;
    a.rec[row] = r;
}

// One part of an unfiltered row (few rows: each is split across `parts`
// workgroups so that the whole GPU streams).  The part's up to kPartTiles
// tiles are loaded together; its maximum and power-of-two sum go to prec,
// and the last of the row's parts to arrive (an arrival counter per row,
// reset by that part) builds the row's record from all of them, so that the
// split costs no launch of its own.
template <int DT>
__device__ __forceinline__ void row_part_plain(const RowArgs& a, RowShared& S, int row, int part) {
    const char* rowp = row_ptr(a.sh, row);
    const int V = a.sh.V;
    const RowStream<DT> st(rowp, V);
    constexpr int NL = RowStream<DT>::NL;
    const int tpp = (st.nt + a.parts - 1) / a.parts;
    const int t0 = part * tpp, n = max(0, min(st.nt, t0 + tpp) - t0);
    float m_th = -INFINITY, k_th = -INFINITY;
    double z_th = 0.0;
    u32x4 raw[kPartTiles][NL];
#pragma unroll
    for (int i = 0; i < kPartTiles; ++i)
        if (i < n) st.issue(t0 + i, raw[i]);
#pragma unroll
    for (int i = 0; i < kPartTiles; ++i) {
        if (i < n) {
            float v[kREPT];
            st.unpack(t0 + i, raw[i], v);
            float tm = v[0];
#pragma unroll
            for (int q = 1; q < kREPT; ++q) tm = fmaxf(tm, v[q]);
            m_th = fmaxf(m_th, tm);
            const float kt = ceilf(tm * a.c8);
            if (kt > k_th) {
                z_th = k_th == -INFINITY ? 0.0 : ldexp(z_th, (int)fmaxf(8.f * (k_th - kt), -4096.f));
                k_th = kt;
            }
            if (k_th != -INFINITY) {
                const float nmc = -8.f * k_th;
                float acc[4];
#pragma unroll
                for (int q = 0; q < kREPT; ++q) {
                    const float term = __builtin_amdgcn_exp2f(fmaf(v[q], a.c_hi, nmc));
                    acc[q & 3] = q < 4 ? term : acc[q & 3] + term;
                }
                z_th += (double)((acc[0] + acc[1]) + (acc[2] + acc[3]));
            }
        }
    }
    const RowTot tot = rb_row_totals(RowTot{m_th, k_th, z_th, 0ull}, S);
    if (threadIdx.x == 0) {
        PartRec* q = a.prec + (size_t)row * a.parts + part;
        __hip_atomic_store(&q->m, tot.m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&q->k, tot.k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&q->z, tot.z, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // the stores are complete before the arrival counts
        unsigned* const cnt = a.part_cnt + (size_t)row * kCntStride;
        const unsigned n = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (n == (unsigned)(a.parts - 1)) {
            merge_row(a, row);
            __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

__global__ void __launch_bounds__(kRB, 4) k_row(RowArgs a) {
    __shared__ RowShared S;
    clear_counters(a.sh);
    // the draw kernel's arrival counters start from zero (it runs after this kernel)
    if (blockIdx.x == 0)
        for (int i = threadIdx.x; i < a.n_cnt; i += kRB) a.draw_cnt[(size_t)i * kCntStride] = 0u;
    if (a.parts > 1) {
        const int row = blockIdx.x / a.parts, part = blockIdx.x % a.parts;
        if (!row_live(a.sh, row)) return;
        if (row_dt(a.sh, row) == DT_BF16)
            row_part_plain<DT_BF16>(a, S, row, part);
        else
            row_part_plain<DT_F32>(a, S, row, part);
        return;
    }
    // With more rows than the GPU holds workgroups at once, the draft rows
    // (the longer streams) go first and the shorter target rows fill the
    // tail; with one round, the target rows go first so that their heavier
    // finalize (kept lists) overlaps the draft rows' streams.
    const int nr = a.sh.n_trows + a.sh.n_drows;
    const int row = a.drafts_first ? (int)((blockIdx.x + (unsigned)a.sh.n_trows) % (unsigned)nr) : (int)blockIdx.x;
    if (!row_live(a.sh, row)) return;  // past its sequence's draft length
    const bool bf = row_dt(a.sh, row) == DT_BF16;
    if (a.use_k) {
        if (bf)
            row_body<DT_BF16, MODE_TOPK>(a, S, row);
        else
            row_body<DT_F32, MODE_TOPK>(a, S, row);
    } else if (a.use_p) {
        if (bf)
            row_body<DT_BF16, MODE_NUCLEUS>(a, S, row);
        else
            row_body<DT_F32, MODE_NUCLEUS>(a, S, row);
    } else {
        if (bf)
            row_body<DT_BF16, MODE_PLAIN>(a, S, row);
        else
            row_body<DT_F32, MODE_PLAIN>(a, S, row);
    }
}

// ---------------------------------------------------------------------------
// k_row_argmax: lowest-index argmax of a target row (greedy mode).
// ---------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ int32_t argmax_body(const Shape& sh, int row, u64* s_red) {
    const char* rowp = row_ptr(sh, row);
    const RowStream<DT> st(rowp, sh.V);
    constexpr int NL = RowStream<DT>::NL;
    float best = -INFINITY;
    int bidx = -1;
    auto process = [&](int t, const u32x4 (&raw)[NL]) {
        float v[kREPT];
        st.unpack(t, raw, v);
        // slots of one thread are in increasing index order across tiles
#pragma unroll
        for (int s = 0; s < kREPT; ++s) {
            const int idx = st.index(t, s);
            if (idx < sh.V && (bidx < 0 || v[s] > best)) {
                best = v[s];
                bidx = idx;
            }
        }
    };
    u32x4 r0[NL], r1[NL];
    st.issue(0, r0);
    for (int t = 0; t < st.nt; t += 2) {
        if (t + 1 < st.nt) st.issue(t + 1, r1);
        process(t, r0);
        if (t + 2 < st.nt) st.issue(t + 2, r0);
        if (t + 1 < st.nt) process(t + 1, r1);
    }
    const u64 key = bidx < 0 ? 0ull
                             : (((u64)fkey(best) << 32) | (u64)(0xFFFFFFFFu - (uint32_t)bidx));
    const u64 k = rb_max_u64(key, s_red);
    return (int32_t)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFull));
}

__global__ void __launch_bounds__(kRB) k_row_argmax(Shape sh, int32_t* gidx) {
    __shared__ u64 s_red[kRW];
    const int row = blockIdx.x;
    clear_counters(sh);
    if (!row_live(sh, row)) return;
    const int32_t g = sh.tdt == DT_BF16 ? argmax_body<DT_BF16>(sh, row, s_red) : argmax_body<DT_F32>(sh, row, s_red);
    if (threadIdx.x == 0) gidx[row] = g;
}

}  // namespace sv
