// spec_verify.hip — C-ABI entry points of the verification library: argument
// checks, per-(device, stream) workspace, kernel launches.
#include <hip/hip_runtime.h>
#include <hip/hip_ext.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/spec_verify.h"
#include "tree_kernels.h"
#include "lmhead_kernels.h"

namespace {

using namespace sv;

// Library-owned scratch for one (device, stream): row records, kept lists of
// filtered target rows (with p and the draft logit of each listed token), greedy
// argmax indices, chunk records and arrival counters of the unfiltered draw,
// the parts of split rows and their arrival counters, and the stops of
// token-tree walks.  Every kernel writes what it later reads within the same
// call.  The draw's arrival counters are cleared by the row kernel before the
// draw runs; the split rows' counters, which the row kernel itself counts
// with (and the single-launch greedy kernel its sequences and batch), sit at
// offset 0 of every layout, are zero when the memory is fresh and are left at
// zero by the workgroup that counts last.
struct Caps {
    size_t rows = 0;         // row records (and split-row partials)
    size_t lists = 0;        // target rows with stored kept lists
    size_t gidx = 0;         // greedy argmax indices
    size_t chunk_bytes = 0;  // chunk records of the unfiltered draw, or the LM-head tile pairs
    size_t seqs = 0;         // sequences: arrival counters and token-tree stops
    size_t nodes = 0;        // token-tree child tokens
    bool covers(const Caps& o) const {
        return o.rows <= rows && o.lists <= lists && o.gidx <= gidx && o.chunk_bytes <= chunk_bytes &&
               o.seqs <= seqs && o.nodes <= nodes;
    }
};

struct Workspace {
    void* base = nullptr;
    Caps cap;
    RowRec* rec = nullptr;
    uint2* kept = nullptr;
    int* kept_n = nullptr;
    float* kept_d = nullptr;
    double* kept_p = nullptr;
    int32_t* gidx = nullptr;
    void* chunks = nullptr;
    unsigned* draw_cnt = nullptr;
    PartRec* prec = nullptr;
    unsigned* part_cnt = nullptr;
    TreeStop* tstop = nullptr;
    int32_t* tex = nullptr;
    int n_cu = 0;  // compute units of the device
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;
void* g_ev_before = nullptr;
void* g_ev_after = nullptr;

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

// Byte offsets of the workspace parts for the capacities c; returns the total.
struct Offsets {
    size_t pc, rec, kept, kn, kd, kp, g, cs, cnt, pr, ts, tx;
};
constexpr size_t kPartCntBytes = (size_t)kSplitRows * kCntStride * sizeof(unsigned);
size_t layout(const Caps& c, Offsets& o) {
    size_t off = 0;
    o.pc = off; off = align_up(off + kPartCntBytes);  // first, at a fixed place
    o.rec = off; off = align_up(off + c.rows * sizeof(RowRec));
    o.kept = off; off = align_up(off + c.lists * (size_t)kListMax * sizeof(uint2));
    o.kn = off; off = align_up(off + c.lists * sizeof(int));
    o.kd = off; off = align_up(off + c.lists * (size_t)kListMax * sizeof(float));
    o.kp = off; off = align_up(off + c.lists * (size_t)kListMax * sizeof(double));
    o.g = off; off = align_up(off + c.gidx * sizeof(int32_t));
    o.cs = off; off = align_up(off + c.chunk_bytes);
    o.cnt = off; off = align_up(off + c.seqs * kCntStride * sizeof(unsigned));
    o.pr = off; off = align_up(off + c.rows * (size_t)kMaxParts * sizeof(PartRec));
    o.ts = off; off = align_up(off + c.seqs * sizeof(TreeStop));
    o.tx = off; off = align_up(off + c.nodes * sizeof(int32_t));
    return std::max<size_t>(off, 256);
}
void carve(char* b, const Caps& c, const Offsets& o, Workspace& w) {
    w.base = b;
    w.cap = c;
    w.rec = reinterpret_cast<RowRec*>(b + o.rec);
    w.kept = reinterpret_cast<uint2*>(b + o.kept);
    w.kept_n = reinterpret_cast<int*>(b + o.kn);
    w.kept_d = reinterpret_cast<float*>(b + o.kd);
    w.kept_p = reinterpret_cast<double*>(b + o.kp);
    w.gidx = reinterpret_cast<int32_t*>(b + o.g);
    w.chunks = b + o.cs;
    w.draw_cnt = reinterpret_cast<unsigned*>(b + o.cnt);
    w.prec = reinterpret_cast<PartRec*>(b + o.pr);
    w.part_cnt = reinterpret_cast<unsigned*>(b + o.pc);
    w.tstop = reinterpret_cast<TreeStop*>(b + o.ts);
    w.tex = reinterpret_cast<int32_t*>(b + o.tx);
}

int get_workspace(hipStream_t stream, const Caps& need, Workspace** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    Workspace& w = g_ws[{dev, stream}];
    if (w.base && w.cap.covers(need)) {
        *out = &w;
        return SPEC_OK;
    }
    Caps c;
    c.rows = std::max(need.rows, w.cap.rows);
    c.lists = std::max(need.lists, w.cap.lists);
    c.gidx = std::max(need.gidx, w.cap.gidx);
    c.chunk_bytes = std::max(need.chunk_bytes, w.cap.chunk_bytes);
    c.seqs = std::max(need.seqs, w.cap.seqs);
    c.nodes = std::max(need.nodes, w.cap.nodes);
    Offsets o;
    const size_t total = layout(c, o);
    if (w.base) {
        // the old buffer may still be in use by work queued on this stream
        if (hipStreamSynchronize(stream) != hipSuccess) return SPEC_E_LAUNCH;
        (void)hipFree(w.base);
        w = Workspace();
    }
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
        return SPEC_E_LAUNCH;
    void* base = nullptr;
    if (hipMalloc(&base, total) != hipSuccess) return SPEC_E_NOMEM;
    if (hipMemsetAsync(base, 0, kPartCntBytes, stream) != hipSuccess) {
        (void)hipFree(base);
        return SPEC_E_LAUNCH;
    }
    Workspace nw;
    carve(static_cast<char*>(base), c, o, nw);
    nw.n_cu = n_cu;
    w = nw;
    *out = &w;
    return SPEC_OK;
}

// ---------------------------------------------------------------------------
// Fixed scratch of the allocation-free entry point: one static device array
// per GPU, held until the process ends.  Host code never uses the array's
// name as an address: each device's address comes from hipGetSymbolAddress,
// taken once with that device current on its first call.
// ---------------------------------------------------------------------------
constexpr size_t kNoAllocBytes = size_t(32) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kNoAllocBytes];

struct NoAllocDevice {
    bool ready = false;
    char* ptr = nullptr;  // device address of `scratch` on this device
    int n_cu = 0;
};
NoAllocDevice g_noalloc[kMaxDevices];

// A workspace carved from the current device's fixed scratch (no allocation).
int noalloc_workspace(const Caps& need, Workspace* w, Workspace** out) {
    Offsets o;
    if (layout(need, o) > kNoAllocBytes) return SPEC_E_SCRATCH;  // checked before any HIP call
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_E_LAUNCH;
    NoAllocDevice& d = g_noalloc[dev];
    {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!d.ready) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SPEC_E_LAUNCH;
            int n_cu = 0;
            if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
                n_cu <= 0)
                return SPEC_E_LAUNCH;
            d.ptr = static_cast<char*>(p);
            d.n_cu = n_cu;
            d.ready = true;
        }
    }
    carve(d.ptr, need, o, *w);
    w->n_cu = d.n_cu;
    *out = w;
    return SPEC_OK;
}

// Where a call's workspace comes from: the per-(device, stream) allocation,
// or (noalloc) the device's fixed scratch, described in `local`.
struct WsSource {
    bool noalloc = false;
    Workspace local;
};
int acquire(hipStream_t stream, const Caps& need, Workspace** out, WsSource* src) {
    if (src && src->noalloc) return noalloc_workspace(need, &src->local, out);
    return get_workspace(stream, need, out);
}

bool dtype_size(int dt, int* sz) {
    if (dt == SPEC_DTYPE_F32) { *sz = 4; return true; }
    if (dt == SPEC_DTYPE_BF16) { *sz = 2; return true; }
    return false;
}

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

int check_sizes(int B, int K, int V) {
    if (B < 0 || K < 0 || V < 1) return SPEC_E_INVALID;
    const long long rows = (long long)B * (2LL * K + 1);
    if (rows >= (1LL << 31)) return SPEC_E_INVALID;
    if (rows * (long long)V >= (1LL << 40)) return SPEC_E_INVALID;
    // a row's byte size (V * 4 for f32 logits) fits the 32-bit size of a raw buffer
    if ((long long)V >= (1LL << 29)) return SPEC_E_INVALID;
    if ((long long)B * ceil_div(V, kChunk) >= (1LL << 31)) return SPEC_E_INVALID;
    return SPEC_OK;
}

int launch_status() { return hipGetLastError() == hipSuccess ? SPEC_OK : SPEC_E_LAUNCH; }

void take_events(void** evb, void** eva) {
    std::lock_guard<std::mutex> lock(g_mu);
    *evb = g_ev_before;
    *eva = g_ev_after;
    g_ev_before = g_ev_after = nullptr;
}

int run_greedy(const void* target, const int32_t* tokens, int B, int K, int V, int32_t* out_tokens,
               int32_t* out_num, hipStream_t stream, int tdt, const int32_t* lens = nullptr,
               int32_t* tested = nullptr, int32_t* accepted = nullptr, WsSource* src = nullptr) {
    int tsz;
    if (!dtype_size(tdt, &tsz)) return SPEC_E_UNSUPPORTED;
    int rc = check_sizes(B, K, V);
    if (rc) return rc;
    if (B == 0) return SPEC_OK;
    if (!target || !out_tokens || !out_num || (K > 0 && !tokens)) return SPEC_E_INVALID;
    const int n_trows = B * (K + 1);
    Workspace* ws;
    Caps need;
    need.gidx = n_trows;
    rc = acquire(stream, need, &ws, src);
    if (rc) return rc;
    const Shape sh{static_cast<const char*>(target), nullptr, tokens, B, K, V, tdt, 0, tsz, 0, n_trows, 0, lens,
                   tested, accepted};
    void *evb, *eva;
    take_events(&evb, &eva);
    if (evb && hipEventRecord(static_cast<hipEvent_t>(evb), stream) != hipSuccess) return SPEC_E_LAUNCH;
    if (B < kSplitRows) {
        // one launch: the last row of each sequence to finish writes its
        // outputs, counted on the split rows' counters (zero between calls)
        const GreedyArgs ga{sh, ws->gidx, out_tokens, out_num, ws->part_cnt};
        hipLaunchKernelGGL(k_greedy_rows, dim3(n_trows), dim3(kRB), 0, stream, ga);
        if ((rc = launch_status())) return rc;
        if (eva && hipEventRecord(static_cast<hipEvent_t>(eva), stream) != hipSuccess) return SPEC_E_LAUNCH;
        return SPEC_OK;
    }
    hipLaunchKernelGGL(k_row_argmax, dim3(n_trows), dim3(kRB), 0, stream, sh, ws->gidx);
    if ((rc = launch_status())) return rc;
    if (eva && hipEventRecord(static_cast<hipEvent_t>(eva), stream) != hipSuccess) return SPEC_E_LAUNCH;
    hipLaunchKernelGGL(k_greedy_prefix, dim3((unsigned)ceil_div(B, 256)), dim3(256), 0, stream, sh,
                       (const int32_t*)ws->gidx, out_tokens, out_num);
    return launch_status();
}

int run_tree_greedy(const void* target, const int32_t* tokens, const int32_t* parents, int B, int N, int V,
                    int32_t* out_tokens, int32_t* out_num, int32_t* out_path, hipStream_t stream, int tdt) {
    int tsz;
    if (!dtype_size(tdt, &tsz)) return SPEC_E_UNSUPPORTED;
    int rc = check_sizes(B, N, V);
    if (rc) return rc;
    if (N > kTreeMax) return SPEC_E_INVALID;
    if (B == 0) return SPEC_OK;
    if (!target || !out_tokens || !out_num || (N > 0 && (!tokens || !parents))) return SPEC_E_INVALID;
    const int n_trows = B * (N + 1);
    Workspace* ws;
    Caps need;
    need.gidx = n_trows;
    rc = get_workspace(stream, need, &ws);
    if (rc) return rc;
    const Shape sh{static_cast<const char*>(target), nullptr, nullptr, B, N, V, tdt, 0, tsz, 0, n_trows, 0,
                   nullptr, nullptr, nullptr};
    void *evb, *eva;
    take_events(&evb, &eva);
    if (evb && hipEventRecord(static_cast<hipEvent_t>(evb), stream) != hipSuccess) return SPEC_E_LAUNCH;
    hipLaunchKernelGGL(k_row_argmax, dim3(n_trows), dim3(kRB), 0, stream, sh, ws->gidx);
    if ((rc = launch_status())) return rc;
    if (eva && hipEventRecord(static_cast<hipEvent_t>(eva), stream) != hipSuccess) return SPEC_E_LAUNCH;
    TreeArgs ta{};
    ta.sh = sh;
    ta.tok = tokens;
    ta.par = parents;
    ta.gidx = ws->gidx;
    ta.out_tokens = out_tokens;
    ta.out_num = out_num;
    ta.out_path = out_path;
    hipLaunchKernelGGL(k_tree_greedy, dim3(B), dim3(64), 0, stream, ta);
    return launch_status();
}

int run_sampling(const void* target, const void* draft, const int32_t* tokens, int B, int K, int V,
                 float temperature, int top_k, float top_p, uint64_t seed, int32_t* out_tokens,
                 int32_t* out_num, hipStream_t stream, int tdt, int ddt, spec_row_stats_t* tstats,
                 spec_row_stats_t* dstats, bool point, const int32_t* lens = nullptr,
                 int32_t* tested = nullptr, int32_t* accepted = nullptr, const int32_t* parents = nullptr,
                 int32_t* out_path = nullptr, WsSource* src = nullptr) {
    // token trees (parents given): K is the node count, tokens the node
    // tokens; the rows carry no token of their own and a walk fixes the stop
    const bool tree = parents != nullptr;
    int tsz, dsz = 4;
    if (!dtype_size(tdt, &tsz)) return SPEC_E_UNSUPPORTED;
    if (K > 0 && !point && !dtype_size(ddt, &dsz)) return SPEC_E_UNSUPPORTED;
    int rc = check_sizes(B, K, V);
    if (rc) return rc;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    const double inv_T = 1.0 / (double)temperature;
    const double c = 1.4426950408889634 / (double)temperature;  // log2(e) / T
    if (!std::isfinite(c) || !(c < 3.0e38)) return SPEC_E_INVALID;
    if (B == 0) return SPEC_OK;
    if (!target || !out_tokens || !out_num) return SPEC_E_INVALID;
    if (K > 0 && ((!point && !draft) || !tokens)) return SPEC_E_INVALID;
    if (point) draft = nullptr;
    if (tree && K > kTreeMax) return SPEC_E_INVALID;

    // point-mass drafts have no draft rows
    const int n_trows = B * (K + 1);
    const int n_drows = point ? 0 : B * K;
    const int rows = n_trows + n_drows;
    const bool use_k = top_k > 0 && top_k < V;
    const bool use_p = top_p < 1.0f;
    const bool filtered = use_k || use_p;
    const int n_chunks = (int)ceil_div(V, kChunk);
    Workspace* ws;
    // drafted sequences with filters draw from kept lists; unfiltered rows
    // and trees draw with chunk sums
    const bool lists = filtered && !tree;
    Caps need;
    need.rows = rows;
    need.lists = lists ? n_trows : 0;
    need.chunk_bytes = lists ? 0 : (size_t)B * n_chunks * sizeof(DrawChunk);
    need.seqs = B;
    need.nodes = tree ? (size_t)B * K : 0;
    rc = acquire(stream, need, &ws, src);
    if (rc) return rc;

    const Shape sh{static_cast<const char*>(target), static_cast<const char*>(draft), tree ? nullptr : tokens,
                   B, K, V, tdt, ddt, tsz, dsz, n_trows, n_drows, lens, tested, accepted};
    RowArgs ra;
    ra.sh = sh;
    // c = c_hi + c_lo with c_hi the largest float below c (so c_hi > 0 and
    // x = -inf gives -inf, never NaN); streamed sums use c_hi, and c_lo
    // corrects them where the exact c's units are needed.
    float c_hi = (float)c;
    if ((double)c_hi >= c) c_hi = std::nextafter(c_hi, 0.0f);
    ra.c_hi = c_hi;
    ra.c_lo = (float)(c - (double)c_hi);
    ra.c64 = c;
    ra.c8 = (float)(c * 0.125);
    ra.inv_T = inv_T;
    ra.top_k = top_k;
    ra.top_p = top_p;
    ra.use_k = use_k;
    ra.use_p = use_p;
    int lg = 0;
    while ((1LL << lg) < (long long)V + 1) ++lg;
    ra.fx_shift = 62 - lg;
    ra.rec = ws->rec;
    ra.kept = ws->kept;
    ra.kept_n = ws->kept_n;
    ra.kept_d = ws->kept_d;
    ra.kept_p = ws->kept_p;
    // A tree's walk needs only the row records; the one stop row per
    // sequence is drawn by the chunked kernels, which read it again.
    ra.want_list = lists ? 1 : 0;
    // two row workgroups fit on a compute unit (their LDS)
    ra.drafts_first = n_drows > 0 && rows > 2 * ws->n_cu ? 1 : 0;
    // Few unfiltered rows: split each across workgroups (at most kPartTiles
    // tiles each) so that about 512 workgroups stream; the last part of each
    // row to finish merges them.
    ra.parts = 1;
    ra.prec = ws->prec;
    ra.part_cnt = ws->part_cnt;
    ra.draw_cnt = ws->draw_cnt;
    ra.n_cnt = B;
    if (!filtered) {
        const int nt = (int)ceil_div(V, kRTile);
        const int want = (int)std::min<long long>(kMaxParts, ceil_div(512, rows));
        const int tpp = (int)ceil_div(nt, std::max(1, want));
        if (want > 1 && tpp <= kPartTiles && rows < kSplitRows) ra.parts = (int)ceil_div(nt, tpp);
    }

    void *evb, *eva;
    take_events(&evb, &eva);
    // with a measurement pair, the events are attached to the dispatch itself
    // (start and end of the kernel, no packets of their own around it)
    hipExtLaunchKernelGGL(k_row, dim3((unsigned)((long long)rows * ra.parts)), dim3(kRB), 0, stream,
                          static_cast<hipEvent_t>(evb), static_cast<hipEvent_t>(eva), 0, ra);
    if ((rc = launch_status())) return rc;

    SeqArgs sa;
    sa.sh = sh;
    sa.inv_T = inv_T;
    sa.seed = seed;
    sa.rec = ws->rec;
    sa.kept = ws->kept;
    sa.kept_n = ws->kept_n;
    sa.kept_d = ws->kept_d;
    sa.kept_p = ws->kept_p;
    sa.chunks = static_cast<DrawChunk*>(ws->chunks);
    sa.draw_cnt = ws->draw_cnt;
    sa.n_chunks = n_chunks;
    sa.out_tokens = out_tokens;
    sa.out_num = out_num;
    sa.point = point ? 1 : 0;
    sa.tstop = nullptr;
    sa.tex = nullptr;
    if (tree) {
        TreeArgs ta;
        ta.sh = sh;
        ta.tok = tokens;
        ta.par = parents;
        ta.inv_T = inv_T;
        ta.seed = seed;
        ta.rec = ws->rec;
        ta.gidx = nullptr;
        ta.tstop = ws->tstop;
        ta.tex = ws->tex;
        ta.out_tokens = out_tokens;
        ta.out_num = out_num;
        ta.out_path = out_path;
        hipLaunchKernelGGL(k_tree_walk, dim3(B), dim3(64), 0, stream, ta);
        if ((rc = launch_status())) return rc;
        sa.tstop = ws->tstop;
        sa.tex = ws->tex;
    }
    if (lists) {
        hipLaunchKernelGGL(k_seq_filtered, dim3((unsigned)((long long)B * (K + 1))), dim3(kSB), 0, stream,
                           sa);
        if ((rc = launch_status())) return rc;
    } else {
        const dim3 g_draw((unsigned)((long long)B * n_chunks));
        if (tree)
            hipLaunchKernelGGL(k_draw<true>, g_draw, dim3(kSB), 0, stream, sa);
        else
            hipLaunchKernelGGL(k_draw<false>, g_draw, dim3(kSB), 0, stream, sa);
        if ((rc = launch_status())) return rc;
    }
    if (tstats || dstats) {
        hipLaunchKernelGGL(k_copy_stats, dim3((unsigned)ceil_div(rows, 256)), dim3(256), 0, stream,
                           (const RowRec*)ws->rec, n_trows, n_drows, tstats, dstats);
        if ((rc = launch_status())) return rc;
    }
    return SPEC_OK;
}

// ---------------------------------------------------------------------------
// The unembedding product (k_lmhead): size checks, arguments, launch.
// ---------------------------------------------------------------------------
int lm_check(long long R, int V, int H) {
    if (R < 0 || V < 1 || H < 8 || H % 8 != 0) return SPEC_E_INVALID;
    const long long n_vt = ceil_div(V, kLmN);
    if (R >= (1LL << 31) || R * n_vt >= (1LL << 40) || (n_vt + 8) * ceil_div(R, kLmM) >= (1LL << 31))
        return SPEC_E_INVALID;
    if ((long long)V * H >= (1LL << 40) || R * H >= (1LL << 40) || R * V >= (1LL << 40)) return SPEC_E_INVALID;
    return SPEC_OK;
}

LmArgs lm_args(const void* hidden, const void* hidden2, long long R1, long long R, const void* w, int V, int H) {
    LmArgs la{};
    la.hidden = static_cast<const uint16_t*>(hidden);
    la.hidden2 = static_cast<const uint16_t*>(hidden2);
    la.R1 = (int)R1;
    la.w = static_cast<const uint16_t*>(w);
    la.R = (int)R;
    la.V = V;
    la.H = H;
    la.n_vt = (int)ceil_div(V, kLmN);
    la.n_rt = (int)ceil_div(R, kLmM);
    return la;
}

// Workgroups of a k_lmhead launch: as many as the GPU holds at once, a
// multiple of 8 (k_lmhead serves the XCDs in turn).
long long lm_grid(int n_cu) { return std::max<long long>(8, (long long)kLmPerCU * n_cu / 8 * 8); }

// Persistent launch: the workgroups the GPU holds at once (a multiple of 8,
// see k_lmhead).  A measurement event pair, if armed, is attached to this
// dispatch.
int launch_lm(int epi, const LmArgs& la, int n_cu, hipStream_t st) {
    const long long grid = lm_grid(n_cu);
    void *evb, *eva;
    take_events(&evb, &eva);
    if (epi == LM_STORE)
        hipExtLaunchKernelGGL(k_lmhead<LM_STORE>, dim3((unsigned)grid), dim3(kLmThreads), 0, st,
                              static_cast<hipEvent_t>(evb), static_cast<hipEvent_t>(eva), 0, la);
    else
        hipExtLaunchKernelGGL(k_lmhead<LM_ARGMAX>, dim3((unsigned)grid), dim3(kLmThreads), 0, st,
                              static_cast<hipEvent_t>(evb), static_cast<hipEvent_t>(eva), 0, la);
    return launch_status();
}

// Compute units of the current device (cached per device).
int device_cus(int* out) {
    static int cus[kMaxDevices] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SPEC_E_LAUNCH;
    if (cus[dev] <= 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
            return SPEC_E_LAUNCH;
        cus[dev] = n;
    }
    *out = cus[dev];
    return SPEC_OK;
}

// The logits of a sampling call from hidden states: one grow-only buffer per
// (device, stream), apart from the verification workspace.
struct LogitBuf {
    void* p = nullptr;
    size_t cap = 0;
};
std::map<std::pair<int, hipStream_t>, LogitBuf> g_lbuf;

int get_logit_buf(hipStream_t stream, size_t bytes, void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SPEC_E_LAUNCH;
    std::lock_guard<std::mutex> lock(g_mu);
    LogitBuf& b = g_lbuf[{dev, stream}];
    if (b.p && bytes <= b.cap) {
        *out = b.p;
        return SPEC_OK;
    }
    if (b.p) {
        if (hipStreamSynchronize(stream) != hipSuccess) return SPEC_E_LAUNCH;
        (void)hipFree(b.p);
        b = LogitBuf();
    }
    if (hipMalloc(&b.p, std::max<size_t>(bytes, 256)) != hipSuccess) {
        b.p = nullptr;
        return SPEC_E_NOMEM;
    }
    b.cap = std::max<size_t>(bytes, 256);
    *out = b.p;
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
                        nullptr, false);
}

int spec_verify_noalloc(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens, int B,
                        int K, int V, float temperature, int top_k, float top_p, uint64_t seed,
                        int32_t* out_tokens, int32_t* out_num_accepted, void* stream, int target_dtype,
                        int draft_dtype) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    WsSource src;
    src.noalloc = true;
    if (temperature == 0.0f)
        return run_greedy(target_logits, draft_tokens, B, K, V, out_tokens, out_num_accepted, s, target_dtype,
                          nullptr, nullptr, nullptr, &src);
    return run_sampling(target_logits, draft_logits, draft_tokens, B, K, V, temperature, top_k, top_p, seed,
                        out_tokens, out_num_accepted, s, target_dtype, draft_dtype, nullptr, nullptr, false,
                        nullptr, nullptr, nullptr, nullptr, nullptr, &src);
}

int spec_verify_point(const void* target_logits, const int32_t* draft_tokens, int B, int K, int V,
                      float temperature, int top_k, float top_p, uint64_t seed, int32_t* out_tokens,
                      int32_t* out_num_accepted, void* stream, int target_dtype) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (temperature == 0.0f)
        return run_greedy(target_logits, draft_tokens, B, K, V, out_tokens, out_num_accepted, s,
                          target_dtype);
    return run_sampling(target_logits, nullptr, draft_tokens, B, K, V, temperature, top_k, top_p, seed,
                        out_tokens, out_num_accepted, s, target_dtype, SPEC_DTYPE_F32, nullptr, nullptr,
                        true);
}

int spec_verify_ragged(const void* target_logits, const void* draft_logits, const int32_t* draft_tokens,
                       const int32_t* draft_lens, int B, int K, int V, float temperature, int top_k,
                       float top_p, uint64_t seed, int32_t* out_tokens, int32_t* out_num_accepted,
                       int32_t* pos_tested, int32_t* pos_accepted, void* stream, int target_dtype,
                       int draft_dtype) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    if (B > 0 && !draft_lens) return SPEC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (temperature == 0.0f)
        return run_greedy(target_logits, draft_tokens, B, K, V, out_tokens, out_num_accepted, s,
                          target_dtype, draft_lens, pos_tested, pos_accepted);
    return run_sampling(target_logits, draft_logits, draft_tokens, B, K, V, temperature, top_k, top_p,
                        seed, out_tokens, out_num_accepted, s, target_dtype, draft_dtype, nullptr,
                        nullptr, false, draft_lens, pos_tested, pos_accepted);
}

int spec_verify_tree(const void* target_logits, const int32_t* node_tokens, const int32_t* parents, int B,
                     int N, int V, float temperature, int top_k, float top_p, uint64_t seed,
                     int32_t* out_tokens, int32_t* out_num_accepted, int32_t* out_path, void* stream,
                     int target_dtype) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    if (N > kTreeMax) return SPEC_E_INVALID;
    if (B > 0 && N > 0 && !parents) return SPEC_E_INVALID;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (temperature == 0.0f)
        return run_tree_greedy(target_logits, node_tokens, parents, B, N, V, out_tokens, out_num_accepted,
                               out_path, s, target_dtype);
    // a tree with no nodes is the bonus draw from the root row: a point-mass
    // call with no drafts (the same row, the same sample counter)
    if (N == 0)
        return run_sampling(target_logits, nullptr, nullptr, B, 0, V, temperature, top_k, top_p, seed, out_tokens,
                            out_num_accepted, s, target_dtype, SPEC_DTYPE_F32, nullptr, nullptr, true);
    return run_sampling(target_logits, nullptr, node_tokens, B, N, V, temperature, top_k, top_p, seed,
                        out_tokens, out_num_accepted, s, target_dtype, SPEC_DTYPE_F32, nullptr, nullptr, true,
                        nullptr, nullptr, nullptr, parents, out_path);
}

int spec_lm_head_logits(const void* hidden, const void* w_unembed, int R, int V, int H, void* out_logits,
                        void* stream) {
    int rc = lm_check(R, V, H);
    if (rc) return rc;
    if (R == 0) return SPEC_OK;
    if (!hidden || !w_unembed || !out_logits) return SPEC_E_INVALID;
    if (((uintptr_t)hidden | (uintptr_t)w_unembed) & 15u) return SPEC_E_INVALID;
    int n_cu;
    if ((rc = device_cus(&n_cu))) return rc;
    LmArgs la = lm_args(hidden, nullptr, R, R, w_unembed, V, H);
    la.logits = static_cast<uint16_t*>(out_logits);
    return launch_lm(LM_STORE, la, n_cu, static_cast<hipStream_t>(stream));
}

int spec_verify_greedy_hidden(const void* hidden, const void* w_unembed, const int32_t* draft_tokens, int B,
                              int K, int V, int H, int32_t* out_tokens, int32_t* out_num_accepted, void* stream) {
    if (B < 0 || K < 0) return SPEC_E_INVALID;
    const long long R = (long long)B * (K + 1);
    if (R >= (1LL << 31)) return SPEC_E_INVALID;
    int rc = lm_check(R, V, H);
    if (rc) return rc;
    if (B == 0) return SPEC_OK;
    if (!hidden || !w_unembed || !out_tokens || !out_num_accepted || (K > 0 && !draft_tokens)) return SPEC_E_INVALID;
    if (((uintptr_t)hidden | (uintptr_t)w_unembed) & 15u) return SPEC_E_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const long long n_vt = ceil_div(V, kLmN);
    Workspace* ws;
    Caps need;
    need.gidx = (size_t)R;
    need.chunk_bytes = (size_t)(R * 2 * n_vt) * sizeof(LmPart);  // one part per tile and wave column
    rc = get_workspace(st, need, &ws);
    if (rc) return rc;
    LmArgs la = lm_args(hidden, nullptr, R, R, w_unembed, V, H);
    la.part = static_cast<LmPart*>(ws->chunks);
    la.gidx = ws->gidx;
    if ((rc = launch_lm(LM_ARGMAX, la, ws->n_cu, st))) return rc;
    const Shape sh{nullptr, nullptr, draft_tokens, B, K, V, SPEC_DTYPE_BF16, 0, 2, 0, (int)R, 0, nullptr, nullptr,
                   nullptr};
    if (B < kSplitRows) {
        // the last merged row of each sequence writes its outputs
        const GreedyArgs ga{sh, ws->gidx, out_tokens, out_num_accepted, ws->part_cnt};
        hipLaunchKernelGGL(k_lmhead_merge_greedy, dim3((unsigned)R), dim3(256), 0, st, la, ga);
        return launch_status();
    }
    hipLaunchKernelGGL(k_lmhead_merge, dim3((unsigned)R), dim3(256), 0, st, la);
    if ((rc = launch_status())) return rc;
    hipLaunchKernelGGL(k_greedy_prefix, dim3((unsigned)ceil_div(B, 256)), dim3(256), 0, st, sh,
                       (const int32_t*)ws->gidx, out_tokens, out_num_accepted);
    return launch_status();
}

int spec_verify_hidden(const void* target_hidden, const void* draft_hidden, const void* w_unembed,
                       const int32_t* draft_tokens, int B, int K, int V, int H, float temperature, int top_k,
                       float top_p, uint64_t seed, int32_t* out_tokens, int32_t* out_num_accepted, void* stream) {
    if (!std::isfinite(temperature) || temperature < 0.0f) return SPEC_E_INVALID;
    if (!(top_p > 0.0f && top_p <= 1.0f)) return SPEC_E_INVALID;
    if (temperature == 0.0f)
        return spec_verify_greedy_hidden(target_hidden, w_unembed, draft_tokens, B, K, V, H, out_tokens,
                                         out_num_accepted, stream);
    if (B < 0 || K < 0) return SPEC_E_INVALID;
    const long long R1 = (long long)B * (K + 1), R = R1 + (long long)B * K;
    if (R >= (1LL << 31)) return SPEC_E_INVALID;
    int rc = lm_check(R, V, H);
    if (rc) return rc;
    if ((rc = check_sizes(B, K, V))) return rc;
    if (B == 0) return SPEC_OK;
    if (!target_hidden || !w_unembed || !out_tokens || !out_num_accepted || (K > 0 && (!draft_hidden || !draft_tokens)))
        return SPEC_E_INVALID;
    if (((uintptr_t)target_hidden | (uintptr_t)w_unembed | (uintptr_t)(K > 0 ? draft_hidden : nullptr)) & 15u)
        return SPEC_E_INVALID;
    hipStream_t st = static_cast<hipStream_t>(stream);
    // the product of every target and draft row with the shared unembedding
    // matrix, in bf16, then the same verification as spec_verify on them
    void* lg = nullptr;
    if ((rc = get_logit_buf(st, (size_t)R * V * sizeof(uint16_t), &lg))) return rc;
    int n_cu;
    if ((rc = device_cus(&n_cu))) return rc;
    LmArgs la = lm_args(target_hidden, draft_hidden, R1, R, w_unembed, V, H);
    la.logits = static_cast<uint16_t*>(lg);
    if ((rc = launch_lm(LM_STORE, la, n_cu, st))) return rc;
    const uint16_t* tl = static_cast<const uint16_t*>(lg);
    return run_sampling(tl, tl + (size_t)R1 * V, draft_tokens, B, K, V, temperature, top_k, top_p, seed, out_tokens,
                        out_num_accepted, st, SPEC_DTYPE_BF16, SPEC_DTYPE_BF16, nullptr, nullptr, false);
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
                        target_dtype, draft_dtype, target_stats, draft_stats, false);
}

int spec_rng_uniforms(uint64_t seed, int B, int K, double* u_accept, double* u_sample,
                      void* stream) {
    if (B < 0 || K < 0 || (long long)B * (K + 1) >= (1LL << 31)) return SPEC_E_INVALID;
    if (B > 0 && !u_sample && !(K > 0 && u_accept)) return SPEC_OK;
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
        case SPEC_E_SCRATCH: return "problem too large for the fixed scratch of the allocation-free entry point";
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
    for (auto& kv : g_lbuf) {
        if (!kv.second.p) continue;
        (void)hipSetDevice(kv.first.first);
        (void)hipStreamSynchronize(kv.first.second);
        (void)hipFree(kv.second.p);
    }
    g_lbuf.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
