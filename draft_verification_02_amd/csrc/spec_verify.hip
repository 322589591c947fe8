// spec_verify.hip — C-ABI entry points of the verification library: argument
// checks, per-(device, stream) workspace, kernel launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/spec_verify.h"
#include "kernels.h"

namespace {

using namespace sv;

// Library-owned scratch for one (device, stream): tile partials, row records,
// sampling chunk sums, counters (kept at zero between calls by the kernels
// that use them) and greedy argmax slots (likewise).
struct Workspace {
    void* base = nullptr;
    size_t bytes = 0;
    size_t cap_tiles = 0, cap_rows = 0, cap_chunks = 0, cap_seqs = 0, cap_trows = 0;
    float* tile_m = nullptr;
    double* tile_z = nullptr;
    RowRec* rec = nullptr;
    double2* chunk_sum = nullptr;
    unsigned* row_cnt = nullptr;
    unsigned* seq_cnt = nullptr;
    unsigned* gseq_cnt = nullptr;
    unsigned long long* gkey = nullptr;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
void* g_ev_before = nullptr;
void* g_ev_after = nullptr;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Returns SPEC_OK and a workspace with at least the requested capacities.
int get_workspace(hipStream_t stream, size_t tiles, size_t rows, size_t chunks, size_t seqs,
                  size_t trows, Workspace** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace& w = g_ws[{dev, stream}];
    if (w.base && tiles <= w.cap_tiles && rows <= w.cap_rows && chunks <= w.cap_chunks &&
        seqs <= w.cap_seqs && trows <= w.cap_trows) {
        *out = &w;
        return SPEC_OK;
    }
    Workspace nw;
    nw.cap_tiles = std::max(tiles, w.cap_tiles);
    nw.cap_rows = std::max(rows, w.cap_rows);
    nw.cap_chunks = std::max(chunks, w.cap_chunks);
    nw.cap_seqs = std::max(seqs, w.cap_seqs);
    nw.cap_trows = std::max(trows, w.cap_trows);
    size_t off = 0;
    const size_t o_tm = off; off = align_up(off + nw.cap_tiles * sizeof(float));
    const size_t o_tz = off; off = align_up(off + nw.cap_tiles * sizeof(double));
    const size_t o_rec = off; off = align_up(off + nw.cap_rows * sizeof(RowRec));
    const size_t o_cs = off; off = align_up(off + nw.cap_chunks * sizeof(double2));
    const size_t o_zero = off;  // counters and slots that must start at zero
    const size_t o_rc = off; off = align_up(off + nw.cap_rows * sizeof(unsigned));
    const size_t o_sc = off; off = align_up(off + nw.cap_seqs * sizeof(unsigned));
    const size_t o_gsc = off; off = align_up(off + nw.cap_seqs * sizeof(unsigned));
    const size_t o_gk = off; off = align_up(off + nw.cap_trows * sizeof(unsigned long long));
    nw.bytes = off;
    if (w.base) {
        // the old buffer may still be in use by work queued on this stream
        if (hipStreamSynchronize(stream) != hipSuccess) return SPEC_E_LAUNCH;
        (void)hipFree(w.base);
        w.base = nullptr;
    }
    if (hipMalloc(&nw.base, nw.bytes) != hipSuccess) {
        w = Workspace();
        return SPEC_E_NOMEM;
    }
    char* b = static_cast<char*>(nw.base);
    if (hipMemsetAsync(b + o_zero, 0, nw.bytes - o_zero, stream) != hipSuccess) {
        (void)hipFree(nw.base);
        w = Workspace();
        return SPEC_E_LAUNCH;
    }
    nw.tile_m = reinterpret_cast<float*>(b + o_tm);
    nw.tile_z = reinterpret_cast<double*>(b + o_tz);
    nw.rec = reinterpret_cast<RowRec*>(b + o_rec);
    nw.chunk_sum = reinterpret_cast<double2*>(b + o_cs);
    nw.row_cnt = reinterpret_cast<unsigned*>(b + o_rc);
    nw.seq_cnt = reinterpret_cast<unsigned*>(b + o_sc);
    nw.gseq_cnt = reinterpret_cast<unsigned*>(b + o_gsc);
    nw.gkey = reinterpret_cast<unsigned long long*>(b + o_gk);
    w = nw;
    *out = &w;
    return SPEC_OK;
}

bool dtype_size(int dt, int* sz) {
    if (dt == SPEC_DTYPE_F32) { *sz = 4; return true; }
    if (dt == SPEC_DTYPE_BF16) { *sz = 2; return true; }
    return false;
}

int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

int check_sizes(int B, int K, int V) {
    if (B < 0 || K < 0 || V < 1) return SPEC_E_INVALID;
    const long long rows = (long long)B * (2LL * K + 1);
    if (rows > (1LL << 30)) return SPEC_E_INVALID;
    if (rows * (long long)V >= (1LL << 40)) return SPEC_E_INVALID;
    if ((long long)V >= (1LL << 31) - kTile) return SPEC_E_INVALID;
    // grid sizes: tiles of every row must fit a 32-bit grid
    if (rows * (long long)ceil_div(V, kTile) >= (1LL << 31)) return SPEC_E_INVALID;
    return SPEC_OK;
}

int launch_status() {
    return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_E_LAUNCH;
}

int run_greedy(const void* target, const int32_t* tokens, int B, int K, int V, int32_t* out_tokens,
               int32_t* out_num, hipStream_t stream, int tdt) {
    int tsz;
    if (!dtype_size(tdt, &tsz)) return SPEC_E_UNSUPPORTED;
    int rc = check_sizes(B, K, V);
    if (rc) return rc;
    if (B == 0) return SPEC_OK;
    if (!target || !out_tokens || !out_num || (K > 0 && !tokens)) return SPEC_E_INVALID;
    const int nt = ceil_div(V, kTile);
    const int n_trows = B * (K + 1);
    Workspace* ws;
    rc = get_workspace(stream, 0, 0, 0, B, n_trows, &ws);
    if (rc) return rc;
    GreedyArgs a;
    a.sh = Shape{static_cast<const char*>(target), nullptr, tokens, B, K, V, tdt, 0, tsz, 0,
                 n_trows, 0, nt};
    a.gkey = ws->gkey;
    a.seq_cnt = ws->gseq_cnt;
    a.out_tokens = out_tokens;
    a.out_num = out_num;
    hipLaunchKernelGGL(k_greedy, dim3((unsigned)((long long)n_trows * nt)), dim3(kBlock), 0, stream, a);
    return launch_status();
}

int run_sampling(const void* target, const void* draft, const int32_t* tokens, int B, int K, int V,
                 float temperature, int top_k, float top_p, uint64_t seed, int32_t* out_tokens,
                 int32_t* out_num, hipStream_t stream, int tdt, int ddt,
                 spec_row_stats_t* tstats, spec_row_stats_t* dstats) {
    int tsz, dsz = 4;
    if (!dtype_size(tdt, &tsz)) return SPEC_E_UNSUPPORTED;
    if (K > 0 && !dtype_size(ddt, &dsz)) return SPEC_E_UNSUPPORTED;
    int rc = check_sizes(B, K, V);
    if (rc) return rc;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    const double inv_T = 1.0 / (double)temperature;
    const double c = 1.4426950408889634 / (double)temperature;  // log2(e) / T
    if (!std::isfinite(c) || !(c < 3.0e38)) return SPEC_E_INVALID;
    if (B == 0) return SPEC_OK;
    if (!target || !out_tokens || !out_num) return SPEC_E_INVALID;
    if (K > 0 && (!draft || !tokens)) return SPEC_E_INVALID;

    const int nt = ceil_div(V, kTile);
    const int n_trows = B * (K + 1);
    const int n_drows = B * K;
    const int rows = n_trows + n_drows;
    const int n_chunks = ceil_div(V, kChunk);
    Workspace* ws;
    rc = get_workspace(stream, (size_t)rows * nt, rows, (size_t)B * n_chunks, B, 0, &ws);
    if (rc) return rc;

    const Shape sh{static_cast<const char*>(target), static_cast<const char*>(draft), tokens, B, K, V,
                   tdt, ddt, tsz, dsz, n_trows, n_drows, nt};
    const bool use_k = top_k > 0 && top_k < V;
    const bool use_p = top_p < 1.0f;

    StreamArgs sa;
    sa.sh = sh;
    // c = c_hi + c_lo with c_hi carrying 12 significant bits, so that
    // (x - M) * c_hi is exact for the 8-bit (bf16) and most f32 differences
    const float c_full = (float)c;
    const float c_hi = __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, c_full) & 0xFFFFF800u);
    sa.c_hi = c_hi;
    sa.c_lo = (float)(c - (double)c_hi);
    sa.inv_T = inv_T;
    sa.filtered = use_k || use_p;
    sa.tile_m = ws->tile_m;
    sa.tile_z = ws->tile_z;
    sa.row_cnt = ws->row_cnt;
    sa.rec = ws->rec;

    void* evb = nullptr;
    void* eva = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        std::swap(evb, g_ev_before);
        std::swap(eva, g_ev_after);
    }
    if (evb && hipEventRecord(static_cast<hipEvent_t>(evb), stream) != hipSuccess) return SPEC_E_LAUNCH;
    hipLaunchKernelGGL(k_rowstats, dim3((unsigned)((long long)rows * nt)), dim3(kBlock), 0, stream, sa);
    if ((rc = launch_status())) return rc;
    if (eva && hipEventRecord(static_cast<hipEvent_t>(eva), stream) != hipSuccess) return SPEC_E_LAUNCH;

    if (sa.filtered) {
        ResolveArgs ra;
        ra.sh = sh;
        ra.inv_T = inv_T;
        ra.top_k = top_k;
        ra.top_p = top_p;
        int lg = 0;
        while ((1LL << lg) < (long long)V + 1) ++lg;
        ra.fx_shift = 62 - lg;
        ra.rec = ws->rec;
        hipLaunchKernelGGL(k_resolve, dim3(rows), dim3(kBlock), 0, stream, ra);
        if ((rc = launch_status())) return rc;
    }

    SampleArgs pa;
    pa.sh = sh;
    pa.inv_T = inv_T;
    pa.seed = seed;
    pa.n_chunks = n_chunks;
    pa.rec = ws->rec;
    pa.chunk_sum = ws->chunk_sum;
    pa.seq_cnt = ws->seq_cnt;
    pa.out_tokens = out_tokens;
    pa.out_num = out_num;
    hipLaunchKernelGGL(k_sample, dim3((unsigned)((long long)B * n_chunks)), dim3(kBlock), 0, stream, pa);
    if ((rc = launch_status())) return rc;

    if (tstats || dstats) {
        hipLaunchKernelGGL(k_copy_stats, dim3(ceil_div(rows, 256)), dim3(256), 0, stream,
                           (const RowRec*)ws->rec, n_trows, n_drows, tstats, dstats);
        if ((rc = launch_status())) return rc;
    }
    return SPEC_OK;
}

}  // namespace

extern "C" {

int spec_verify(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                int B, int K, int V, float temperature, int top_k, float top_p, uint64_t seed,
                int32_t* out_tokens, int32_t* out_num_accepted, void* stream, int target_dtype,
                int draft_dtype) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (temperature == 0.0f)
        return run_greedy(target_logits, draft_tokens, B, K, V, out_tokens, out_num_accepted, s,
                          target_dtype);
    return run_sampling(target_logits, draft_logits, draft_tokens, B, K, V, temperature, top_k, top_p,
                        seed, out_tokens, out_num_accepted, s, target_dtype, draft_dtype, nullptr,
                        nullptr);
}

int spec_verify_greedy(const void* target_logits, const int32_t* draft_tokens, int B, int K, int V,
                       int32_t* out_tokens, int32_t* out_num_accepted, void* stream,
                       int target_dtype) {
    return run_greedy(target_logits, draft_tokens, B, K, V, out_tokens, out_num_accepted,
                      static_cast<hipStream_t>(stream), target_dtype);
}

int spec_verify_stats(const void* target_logits, const void* draft_logits,
                      const int32_t* draft_tokens, int B, int K, int V, float temperature, int top_k,
                      float top_p, uint64_t seed, int32_t* out_tokens, int32_t* out_num_accepted,
                      void* stream, int target_dtype, int draft_dtype,
                      spec_row_stats_t* target_stats, spec_row_stats_t* draft_stats) {
    if (!std::isfinite(temperature) || !(temperature > 0.0f)) return SPEC_E_INVALID;
    return run_sampling(target_logits, draft_logits, draft_tokens, B, K, V, temperature, top_k, top_p,
                        seed, out_tokens, out_num_accepted, static_cast<hipStream_t>(stream),
                        target_dtype, draft_dtype, target_stats, draft_stats);
}

int spec_rng_uniforms(uint64_t seed, int B, int K, double* u_accept, double* u_sample,
                      void* stream) {
    if (B < 0 || K < 0 || (long long)B * (K + 1) >= (1LL << 31)) return SPEC_E_INVALID;
    if (B == 0) return SPEC_OK;
    const long long n = (long long)B * (K + 1);
    hipLaunchKernelGGL(k_uniforms, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                       static_cast<hipStream_t>(stream), seed, B, K, u_accept, u_sample);
    return launch_status();
}

int spec_profile_events(void* before, void* after) {
    std::lock_guard<std::mutex> lock(g_mu);
    if (before && after) {
        g_ev_before = before;
        g_ev_after = after;
    } else {
        g_ev_before = nullptr;
        g_ev_after = nullptr;
    }
    return SPEC_OK;
}

const char* spec_status_string(int status) {
    switch (status) {
        case SPEC_OK: return "ok";
        case SPEC_E_INVALID: return "invalid argument";
        case SPEC_E_UNSUPPORTED: return "unsupported dtype";
        case SPEC_E_NOMEM: return "workspace allocation failed";
        case SPEC_E_LAUNCH: return "HIP runtime or kernel launch failure";
        default: return "unknown status";
    }
}

void spec_release_workspace(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto& kv : g_ws) {
        if (!kv.second.base) continue;
        (void)hipSetDevice(kv.first.first);
        (void)hipStreamSynchronize(kv.first.second);
        (void)hipFree(kv.second.base);
    }
    g_ws.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
