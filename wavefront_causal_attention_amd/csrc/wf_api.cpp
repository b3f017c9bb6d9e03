// C ABI of the wavefront-round attention library: validation, the round
// schedule, readiness bookkeeping and the page-table closed form. Every device
// step is a kernel launched through wf_internal.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <vector>

#include "../../include/wf.h"
#include "wf_internal.h"

namespace {

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

// Byte layout of the caller's pool allocation.
struct Layout {
    int N = 0, T = 0, R = 0, ppc = 0, nblk = 0;
    size_t k_layer = 0, v_layer = 0;       // bytes per layer
    size_t k_off = 0, v_off = 0;           // region offsets
    size_t scale_off = 0, mean_off = 0, part_off = 0;        // fp8 metadata and publish scratch
    size_t scale_layer = 0, mean_layer = 0, part_layer = 0;
    size_t htab_off = 0, wtab_off = 0, omega_off = 0;
    size_t htab64_off = 0, wtab64_off = 0; // fp64 (cos, sin) row / column tables of the publish
    size_t ring_off = 0;                   // device round counter (int64): advances since creation
    size_t work_off = 0, work_stride = 0;  // attention work lists, one per slot range
    int work_len = 0;                      // entries per list
    size_t pool_bytes = 0, table_bytes = 0;
};

// Attention work order for query slots [first, first + n): every (slot, head,
// query tile) unit, cost = key chunks it reads (for packing, the run-time
// estimate pcost, which discounts a mostly idle last query tile). Units are laid out head-major
// and cut into kXcds contiguous pieces of equal cost (each unit goes to the
// piece holding its cost midpoint), so one head's K/V is streamed by one or
// two XCDs (each XCD has its own L2). Workgroup b runs piece b % kXcds, entry
// b / kXcds. Returns the padded list.
//
// Inside a piece the order serves the hardware dispatcher, which hands the
// next workgroup to the first CU that frees up (one workgroup per CU here):
// the units are first packed onto the XCD's CUs (longest first onto the least
// loaded CU, then moves and swaps that lower the most loaded CU), and then
// emitted by their planned start times, so that dispatch replays the packing
// when run times follow the cost model and still adapts when they do not.
struct WorkUnit {
    int s, h, q;
    int64_t cost;     // key chunks x 10: cuts the list into XCD pieces
    int64_t pcost;    // run-time estimate used to pack a piece onto CUs
};

static void order_piece(std::vector<WorkUnit>& p, int bins) {
    const int n = (int)p.size();
    std::vector<int> idx(n);
    for (int i = 0; i < n; ++i) idx[i] = i;
    std::stable_sort(idx.begin(), idx.end(), [&](int x, int y) { return p[x].pcost > p[y].pcost; });
    if (bins <= 1 || n <= 1) {
        std::vector<WorkUnit> out;
        for (int i : idx) out.push_back(p[i]);
        p.swap(out);
        return;
    }
    std::vector<std::vector<int>> bin(bins);
    std::vector<int64_t> load(bins, 0);
    for (int i : idx) {
        const int b = (int)(std::min_element(load.begin(), load.end()) - load.begin());
        bin[b].push_back(i);
        load[b] += p[i].pcost;
    }
    // descent on the most loaded bin; every accepted move or swap makes the
    // pair's loads more even, so the sum of squared loads strictly falls
    std::vector<int> by_load(bins);
    for (int iter = 0; iter < 100000; ++iter) {
        const int hi = (int)(std::max_element(load.begin(), load.end()) - load.begin());
        for (int b = 0; b < bins; ++b) by_load[b] = b;
        std::stable_sort(by_load.begin(), by_load.end(), [&](int x, int y) { return load[x] < load[y]; });
        bool moved = false;
        for (int lo : by_load) {
            if (lo == hi) continue;
            int64_t best = load[hi];
            int bi = -1, bj = -1;
            for (size_t i = 0; i < bin[hi].size(); ++i) {
                const int64_t ci = p[bin[hi][i]].pcost;
                if (std::max(load[hi] - ci, load[lo] + ci) < best) {
                    best = std::max(load[hi] - ci, load[lo] + ci);
                    bi = (int)i;
                    bj = -1;
                }
                for (size_t j = 0; j < bin[lo].size(); ++j) {
                    const int64_t d = ci - p[bin[lo][j]].pcost;
                    if (d > 0 && std::max(load[hi] - d, load[lo] + d) < best) {
                        best = std::max(load[hi] - d, load[lo] + d);
                        bi = (int)i;
                        bj = (int)j;
                    }
                }
            }
            if (bi < 0) continue;
            const int ui = bin[hi][bi];
            if (bj < 0) {
                bin[hi].erase(bin[hi].begin() + bi);
                bin[lo].push_back(ui);
                load[hi] -= p[ui].pcost;
                load[lo] += p[ui].pcost;
            } else {
                const int uj = bin[lo][bj];
                bin[hi][bi] = uj;
                bin[lo][bj] = ui;
                load[hi] += p[uj].pcost - p[ui].pcost;
                load[lo] += p[ui].pcost - p[uj].pcost;
            }
            moved = true;
            break;
        }
        if (!moved) break;
    }
    // planned start times: each CU runs its units longest first
    struct Start { int64_t t, neg_cost; int i; };
    std::vector<Start> st;
    st.reserve(n);
    for (auto& b : bin) {
        std::stable_sort(b.begin(), b.end(), [&](int x, int y) { return p[x].pcost > p[y].pcost; });
        int64_t t = 0;
        for (int i : b) {
            st.push_back({t, -p[i].pcost, i});
            t += p[i].pcost;
        }
    }
    std::sort(st.begin(), st.end(), [](const Start& x, const Start& y) {
        return x.t != y.t ? x.t < y.t : x.neg_cost != y.neg_cost ? x.neg_cost < y.neg_cost : x.i < y.i;
    });
    std::vector<WorkUnit> out;
    out.reserve(n);
    for (const Start& x : st) out.push_back(p[x.i]);
    p.swap(out);
}

// cus_per_xcd <= 0 skips the ordering (list sizes do not depend on it).
std::vector<int32_t> build_work_list(int first, int n, int heads, int N, int T, bool all_live, bool fp8,
                                     int cus_per_xcd) {
    const int qtiles = (N + wf::kAttnBM - 1) / wf::kAttnBM;
    // costs in tenths of a key chunk. The last query tile, when at most half
    // its waves hold rows of the chunk, runs one computing wave per SIMD (the
    // others idle): for bf16, packing counts it as 0.6 of a full tile (0.6,
    // 0.7 and 0.8 measured at three Wan shapes; 0.6 was never slower than
    // 1.0). The fp8 kernel's tail tiles measured no faster, so fp8 keeps whole
    // tiles, as does the XCD cut.
    const int tail_waves = (N - (qtiles - 1) * wf::kAttnBM + 31) / 32;
    const int64_t tail_w = !fp8 && tail_waves <= wf::kAttnBM / 64 ? 6 : 10;
    std::vector<WorkUnit> u;
    u.reserve((size_t)n * heads * qtiles);
    for (int h = 0; h < heads; ++h)
        for (int s = first; s < first + n; ++s)
            for (int q = 0; q < qtiles; ++q)
                u.push_back({s, h, q, (int64_t)(all_live ? T : T - s) * 10,
                             (int64_t)(all_live ? T : T - s) * (q == qtiles - 1 ? tail_w : 10)});
    int64_t total = 0;
    for (const WorkUnit& x : u) total += x.cost;
    std::vector<std::vector<WorkUnit>> piece(wf::kXcds);
    int64_t acc = 0;
    for (const WorkUnit& x : u) {
        int xcd = (int)((2 * acc + x.cost) * wf::kXcds / std::max<int64_t>(2 * total, 1));
        xcd = std::min(std::max(xcd, 0), wf::kXcds - 1);
        piece[xcd].push_back(x);
        acc += x.cost;
    }
    size_t M = 0;
    for (auto& p : piece) {
        if (cus_per_xcd > 0) order_piece(p, cus_per_xcd);
        M = std::max(M, p.size());
    }
    std::vector<int32_t> out(M * wf::kXcds, wf::kIdleWork);
    for (int x = 0; x < wf::kXcds; ++x)
        for (size_t j = 0; j < piece[x].size(); ++j)
            out[j * wf::kXcds + x] = wf::pack_work(piece[x][j].s, piece[x][j].h, piece[x][j].q);
    return out;
}

int validate(const wf_config* c, Layout* L) {
    if (!c) return WF_E_INVALID_ARG;
    if (c->S < 1 || c->anchor_chunks < 1 || c->history_chunks < 0) return WF_E_SHAPE;
    const int T = c->anchor_chunks + c->history_chunks + c->S + 1;
    if (T > wf::kMaxSlots) return WF_E_SHAPE;
    if (c->heads < 1 || c->heads > 1024) return WF_E_SHAPE;
    if (c->head_dim != 64 && c->head_dim != 128) return WF_E_SHAPE;
    if (c->num_layers < 1 || c->num_layers > 4096) return WF_E_SHAPE;
    if (c->chunk_frames < 1 || c->frame_h < 1 || c->frame_w < 1) return WF_E_SHAPE;
    const int64_t N = (int64_t)c->chunk_frames * c->frame_h * c->frame_w;
    if (N > (1 << 20)) return WF_E_SHAPE;
    // attention splits flat context keys into page and token in fp32, exact
    // below 2^22 - 1 keys
    if ((int64_t)T * N >= (1 << 22) - 1) return WF_E_SHAPE;
    if (c->page_tokens < 8 || c->page_tokens % 8 != 0 || N % c->page_tokens != 0) return WF_E_SHAPE;
    // fp8 attention tiles each chunk into its 64-token quantisation blocks and
    // stages one key scale per tile of the context in LDS
    if (c->qk_dtype == WF_DTYPE_FP8_E4M3 && (int64_t)T * ((N + 63) / 64) > wf::kMaxFp8Tiles)
        return WF_E_SHAPE;
    const int ppc = (int)(N / c->page_tokens);
    if ((int64_t)T * ppc > wf::kMaxTablePages) return WF_E_SHAPE;
    if (c->in_dtype != WF_DTYPE_BF16 && c->in_dtype != WF_DTYPE_FP32) return WF_E_INVALID_ARG;
    if (c->qk_dtype != WF_DTYPE_BF16 && c->qk_dtype != WF_DTYPE_FP8_E4M3) return WF_E_INVALID_ARG;
    if (c->live_mask != WF_MASK_WAVEFRONT && c->live_mask != WF_MASK_ALL_LIVE) return WF_E_INVALID_ARG;
    const int dt = c->rope_split[0], dh = c->rope_split[1], dw = c->rope_split[2];
    if (dt < 0 || dh < 0 || dw < 0 || (dt | dh | dw) & 1 || dt + dh + dw != c->head_dim) return WF_E_SHAPE;
    if (dt > 64) return WF_E_SHAPE;
    if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta)) return WF_E_INVALID_ARG;
    if (c->first_round < 0 || c->total_chunks < 0) return WF_E_SHAPE;
    if (c->total_chunks > 0 && (int64_t)c->first_round > (int64_t)c->total_chunks - 1 + c->S) return WF_E_SHAPE;
    if ((int64_t)c->first_round + 1000000000LL > INT32_MAX / std::max(1, c->chunk_frames)) {
        // keep chunk_frames * chunk id representable for a very long stream
        if ((int64_t)c->chunk_frames * (c->first_round + 1) > INT32_MAX / 2) return WF_E_SHAPE;
    }
    if (!L) return WF_OK;
    const bool fp8 = c->qk_dtype == WF_DTYPE_FP8_E4M3;
    L->N = (int)N;
    L->T = T;
    L->R = c->history_chunks + c->S + 1;
    L->ppc = ppc;
    L->nblk = (int)((N + wf::kFp8Block - 1) / wf::kFp8Block);
    const size_t pages = (size_t)T * ppc;
    const size_t elems = pages * c->heads * c->page_tokens * (size_t)c->head_dim;
    L->k_layer = align_up(elems * (fp8 ? 1 : 2), 256);
    L->v_layer = align_up(elems * 2, 256);
    if (L->k_layer >= (1ull << 31) || L->v_layer >= (1ull << 31)) return WF_E_SHAPE;  // 32-bit buffer offsets
    size_t off = 0;
    L->k_off = off;  off += L->k_layer * c->num_layers;
    L->v_off = off;  off += L->v_layer * c->num_layers;
    if (fp8) {
        // K scale per token (its 64-token block's scale, replicated), K mean
        // per (group, head), and the publish's scratch: the fp64 sums of
        // RoPE'd K per (published slot, head, 64-token block)
        L->scale_layer = align_up(pages * c->heads * c->page_tokens * 4, 256);
        L->mean_layer = align_up((size_t)T * c->heads * c->head_dim * 4, 256);
        L->part_layer = align_up((size_t)T * c->heads * L->nblk * c->head_dim * 8, 256);
        if (L->scale_layer >= (1ull << 31)) return WF_E_SHAPE;
        L->scale_off = off;  off += L->scale_layer * c->num_layers;
        L->mean_off = off;   off += L->mean_layer * c->num_layers;
        L->part_off = off;   off += L->part_layer * c->num_layers;
    }
    L->htab_off = off;  off += align_up((size_t)c->frame_h * (dh / 2) * 8 + 8, 256);
    L->wtab_off = off;  off += align_up((size_t)c->frame_w * (dw / 2) * 8 + 8, 256);
    L->htab64_off = off;  off += align_up((size_t)c->frame_h * (dh / 2) * 16 + 16, 256);
    L->wtab64_off = off;  off += align_up((size_t)c->frame_w * (dw / 2) * 16 + 16, 256);
    L->omega_off = off; off += align_up((size_t)(dt / 2) * 8 + 8, 256);
    L->ring_off = off;  off += 256;
    {
        const int qtiles = (int)((N + wf::kAttnBM - 1) / wf::kAttnBM);
        const int64_t units = (int64_t)(c->S + 1) * c->heads * qtiles;
        if (units >= (1 << 22) || qtiles > 0xFFFF) return WF_E_SHAPE;
        size_t longest = 0;
        for (int first = 0; first <= c->S; ++first)
            for (int n = 1; first + n <= c->S + 1; ++n)
                longest = std::max(longest, build_work_list(first, n, c->heads, (int)N, T,
                                                            c->live_mask == WF_MASK_ALL_LIVE, fp8, 0).size());
        L->work_len = (int)longest;
        L->work_stride = align_up(longest * 4, 256);
        L->work_off = off;
        off += L->work_stride * (size_t)(c->S + 1) * (c->S + 1);
    }
    L->pool_bytes = off;
    L->table_bytes = pages * sizeof(int32_t);
    return WF_OK;
}

}  // namespace

struct wf_handle {
    wf_config cfg;
    Layout L;
    bool host_model = false;
    char* pool = nullptr;
    int32_t* table = nullptr;
    int64_t ring = 0;                    // advances since creation
    bool captured = false;               // an advance of this pool was captured into a graph
    std::vector<uint64_t> ready;         // per layer, bit p = context position p
    std::vector<int> work_count;         // attention work-list length per slot range
    char err[512] = {0};

    int A() const { return cfg.anchor_chunks; }
    int H() const { return cfg.history_chunks; }
    int S() const { return cfg.S; }
    int64_t round() const { return cfg.first_round + ring; }
    int position_of_slot(int s) const { return L.T - 1 - s; }

    // Chunk id at context position p in round k (k = i + s).
    int64_t chunk_at_round(int p, int64_t k) const {
        if (p < A()) return p;
        if (p < A() + H()) return k - S() - H() + (p - A());
        const int s = L.T - 1 - p;       // live slot index, store = S
        return k - s;
    }
    int64_t chunk_at(int p) const { return chunk_at_round(p, round()); }
    // Whether position p holds a chunk in round k: chunk i is stored in round
    // i + S and clean afterwards (anchor chunks at the anchor, later ones in
    // the history ring); C = total_chunks bounds the video when positive.
    bool present_at_round(int p, int64_t k) const {
        const int64_t c = chunk_at_round(p, k);
        const bool in_video = cfg.total_chunks <= 0 || c <= (int64_t)cfg.total_chunks - 1;
        if (p < A()) return k >= c + S() + 1 && in_video;
        if (p < A() + H()) return c >= A() && in_video;
        return c >= 0 && in_video;
    }
    bool present(int p) const { return present_at_round(p, round()); }
    // Anchor chunk held by the store in round k, or -1: it is published
    // straight into that anchor's pages.
    int store_anchor_at_round(int64_t k) const {
        const int64_t c = k - S();
        return present_at_round(A() + H(), k) && c < A() ? (int)c : -1;
    }
    // Page group of context position p: the anchor is fixed; the ring of
    // H+S+1 groups rotates by one per advance; a store holding an anchor
    // chunk writes that anchor's group.
    int group_at(int p) const {
        if (p < A()) return p;
        if (p == A() + H()) {
            const int a = store_anchor_at_round(round());
            if (a >= 0) return a;
        }
        return A() + (int)(((int64_t)(p - A()) + ring) % L.R);
    }
    uint64_t prefix_bits(int n) const { return n >= 64 ? ~0ull : ((1ull << n) - 1); }
    int64_t* ring_dev() const { return host_model ? nullptr : (int64_t*)(pool + L.ring_off); }
    // every position holds a chunk and the store holds no anchor chunk
    bool steady_at_round(int64_t k) const {
        for (int p = 0; p < L.T; ++p)
            if (!present_at_round(p, k)) return false;
        return store_anchor_at_round(k) < 0;
    }

    int fail_hip(hipError_t e, const char* what) {
        snprintf(err, sizeof err, "%s: %s", what, hipGetErrorString(e));
        return WF_E_HIP;
    }
};

extern "C" {

int wf_pool_bytes(const wf_config* cfg, size_t* pool_bytes, size_t* table_bytes) {
    if (!pool_bytes || !table_bytes) return WF_E_INVALID_ARG;
    Layout L;
    const int st = validate(cfg, &L);
    if (st != WF_OK) return st;
    *pool_bytes = L.pool_bytes;
    *table_bytes = L.table_bytes;
    return WF_OK;
}

static int make_handle(const wf_config* cfg, wf_handle** out, Layout* L) {
    if (!out) return WF_E_INVALID_ARG;
    const int st = validate(cfg, L);
    if (st != WF_OK) return st;
    wf_handle* h = new (std::nothrow) wf_handle();
    if (!h) return WF_E_INVALID_ARG;
    h->cfg = *cfg;
    h->L = *L;
    h->ready.assign(cfg->num_layers, 0);
    h->work_count.assign((size_t)(cfg->S + 1) * (cfg->S + 1), 0);
    *out = h;
    return WF_OK;
}

int wf_pool_create_host_model(const wf_config* cfg, wf_handle** out) {
    Layout L;
    wf_handle* h = nullptr;
    const int st = make_handle(cfg, &h, &L);
    if (st != WF_OK) return st;
    h->host_model = true;
    *out = h;
    return WF_OK;
}

int wf_pool_create(const wf_config* cfg, void* pool_dev, size_t pool_bytes,
                   int32_t* page_table_dev, size_t table_bytes, wf_handle** out) {
    if (!pool_dev || !page_table_dev || !out) return WF_E_INVALID_ARG;
    Layout L;
    int st = validate(cfg, &L);
    if (st != WF_OK) return st;
    if (pool_bytes < L.pool_bytes || table_bytes < L.table_bytes) return WF_E_SHAPE;
    if (((uintptr_t)pool_dev & 255) || ((uintptr_t)page_table_dev & 3)) return WF_E_INVALID_ARG;
    wf_handle* h = nullptr;
    st = make_handle(cfg, &h, &L);
    if (st != WF_OK) return st;
    h->pool = (char*)pool_dev;
    h->table = page_table_dev;

    // RoPE tables, fp64 on the host, stored as fp32 (cos, sin) for the row and
    // column axes; the time axis keeps fp64 frequencies because its positions
    // grow with the stream and are expanded per launch.
    const int dt = cfg->rope_split[0], dh = cfg->rope_split[1], dw = cfg->rope_split[2];
    // The publish kernels rotate in fp64 and take the fp64 tables; the fused
    // projection rotates its fp32 accumulators with the fp32 ones.
    std::vector<double> htab64((size_t)cfg->frame_h * (dh / 2) * 2 + 2, 0.0);
    std::vector<double> wtab64((size_t)cfg->frame_w * (dw / 2) * 2 + 2, 0.0);
    std::vector<double> om((size_t)(dt / 2) + 1, 0.0);
    for (int y = 0; y < cfg->frame_h; ++y)
        for (int m = 0; m < dh / 2; ++m) {
            const double phi = y * std::pow(cfg->rope_theta, -2.0 * m / dh);
            htab64[((size_t)y * (dh / 2) + m) * 2 + 0] = std::cos(phi);
            htab64[((size_t)y * (dh / 2) + m) * 2 + 1] = std::sin(phi);
        }
    for (int x = 0; x < cfg->frame_w; ++x)
        for (int m = 0; m < dw / 2; ++m) {
            const double phi = x * std::pow(cfg->rope_theta, -2.0 * m / dw);
            wtab64[((size_t)x * (dw / 2) + m) * 2 + 0] = std::cos(phi);
            wtab64[((size_t)x * (dw / 2) + m) * 2 + 1] = std::sin(phi);
        }
    for (int m = 0; m < dt / 2; ++m) om[m] = std::pow(cfg->rope_theta, -2.0 * m / dt);
    std::vector<float> htab(htab64.size()), wtab(wtab64.size());
    for (size_t i = 0; i < htab64.size(); ++i) htab[i] = (float)htab64[i];
    for (size_t i = 0; i < wtab64.size(); ++i) wtab[i] = (float)wtab64[i];

    // the static scratch of wf_kv_publish_noalloc, looked up once per device
    void* sptr = nullptr;
    hipError_t e = wf::static_scratch(&sptr);
    if (e == hipSuccess) e = hipMemcpy(h->pool + L.htab_off, htab.data(), htab.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->pool + L.wtab_off, wtab.data(), wtab.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->pool + L.htab64_off, htab64.data(), htab64.size() * 8, hipMemcpyHostToDevice);
    if (e == hipSuccess)
        e = hipMemcpy(h->pool + L.wtab64_off, wtab64.data(), wtab64.size() * 8, hipMemcpyHostToDevice);

    if (e == hipSuccess)
        e = hipMemcpy(h->pool + L.omega_off, om.data(), om.size() * 8, hipMemcpyHostToDevice);
    const int64_t ring0 = 0;
    if (e == hipSuccess) e = hipMemcpy(h->pool + L.ring_off, &ring0, sizeof ring0, hipMemcpyHostToDevice);
    const int qtiles = (L.N + wf::kAttnBM - 1) / wf::kAttnBM;
    int cus = 0;
    if (e == hipSuccess) {
        int dev = 0;
        e = hipGetDevice(&dev);
        if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    }
    const int cus_per_xcd = std::max(1, cus / wf::kXcds);
    for (int first = 0; first <= cfg->S && e == hipSuccess; ++first)
        for (int n = 1; first + n <= cfg->S + 1 && e == hipSuccess; ++n) {
            std::vector<int32_t> wl = build_work_list(first, n, cfg->heads, L.N, L.T,
                                                      cfg->live_mask == WF_MASK_ALL_LIVE,
                                                      cfg->qk_dtype == WF_DTYPE_FP8_E4M3, cus_per_xcd);
            if ((int)wl.size() > L.work_len) { e = hipErrorInvalidValue; break; }
            h->work_count[first * (cfg->S + 1) + n - 1] = (int)wl.size();
            e = hipMemcpy(h->pool + L.work_off + L.work_stride * (first * (cfg->S + 1) + n - 1),
                          wl.data(), wl.size() * 4, hipMemcpyHostToDevice);
        }
    if (e == hipSuccess)
        e = wf::launch_page_table(h->table, L.T, cfg->anchor_chunks, L.ppc, h->ring, nullptr,
                                  cfg->anchor_chunks + cfg->history_chunks,
                                  h->store_anchor_at_round(h->round()), nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
        delete h;
        return WF_E_HIP;
    }
    *out = h;
    return WF_OK;
}

void wf_pool_destroy(wf_handle* h) { delete h; }

// The publish; static_scratch: the fp8 K-mean block sums go to the library's
// static per-GPU array instead of the pool's scratch region.
static int publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots, const void* q, const void* k,
                   const void* v, int64_t row_stride_elems, const int32_t* chunk_t0_host, void* q_out,
                   float* q_scales, void* stream, bool static_scratch) {
    if (!h) return WF_E_INVALID_ARG;
    const wf_config& c = h->cfg;
    const Layout& L = h->L;
    if (layer < 0 || layer >= c.num_layers) return WF_E_INVALID_ARG;
    if (nslots < 1 || slot_first < 0 || slot_first + nslots > L.T) return WF_E_INVALID_ARG;
    if (!k || !v) return WF_E_INVALID_ARG;
    if (row_stride_elems < (int64_t)c.heads * c.head_dim) return WF_E_INVALID_ARG;
    if ((q == nullptr) != (q_out == nullptr)) return WF_E_INVALID_ARG;
    if (q && slot_first + nslots > c.S + 1) return WF_E_INVALID_ARG;
    const bool fp8 = c.qk_dtype == WF_DTYPE_FP8_E4M3;
    if (fp8 && q_out && !q_scales) return WF_E_INVALID_ARG;
    const int esz = c.in_dtype == WF_DTYPE_FP32 ? 4 : 2;
    if (((uintptr_t)k | (uintptr_t)v | (uintptr_t)q) % (esz * 8) ||
        (row_stride_elems * esz) % 16)
        return WF_E_INVALID_ARG;      // 8-element vector loads
    if (q_out && ((uintptr_t)q_out % 16)) return WF_E_INVALID_ARG;

    for (int i = 0; i < nslots; ++i)
        if (!h->present(h->position_of_slot(slot_first + i))) {
            snprintf(h->err, sizeof h->err, "slot %d holds no chunk in round %lld", slot_first + i,
                     (long long)h->round());
            return WF_E_INVALID_ARG;
        }
    // fp8: K-mean block sums of the published slots, fp64
    const size_t part_bytes = fp8 ? (size_t)nslots * c.heads * L.nblk * c.head_dim * 8 : 0;
    if (static_scratch && part_bytes > wf::kStaticScratchBytes) {
        snprintf(h->err, sizeof h->err, "wf_kv_publish_noalloc: %zu scratch bytes needed, the static array holds %zu",
                 part_bytes, wf::kStaticScratchBytes);
        return WF_E_SHAPE;
    }
    void* sptr = nullptr;
    if (static_scratch && fp8 && !h->host_model) {
        const hipError_t e = wf::static_scratch(&sptr);
        if (e != hipSuccess) return h->fail_hip(e, "wf_kv_publish_noalloc scratch address");
    }
    wf::PublishArgs a{};
    for (int i = 0; i < nslots; ++i) {
        const int64_t t0 = chunk_t0_host
                               ? (int64_t)chunk_t0_host[i]
                               : (int64_t)c.chunk_frames * h->chunk_at(h->position_of_slot(slot_first + i));
        if (t0 < 0 || t0 > INT32_MAX / 2) return WF_E_INVALID_ARG;
        a.t0[i] = (int)t0;
    }
    // live slots take their chunk id from the device round counter (the same
    // values in eager use; right in every round a captured launch replays)
    if (!chunk_t0_host && slot_first + nslots <= c.S + 1) {
        a.ring = h->ring_dev();
        a.t0_round = c.first_round - slot_first;
        a.chunk_frames = c.chunk_frames;
    }
    if (!h->host_model) {
        a.q = q; a.k = k; a.v = v;
        a.row_stride = row_stride_elems;
        a.q_out = q_out;
        a.q_scales = q_scales;
        a.kpage = h->pool + L.k_off + L.k_layer * layer;
        a.vpage = (uint16_t*)(h->pool + L.v_off + L.v_layer * layer);
        a.kscale = fp8 ? (float*)(h->pool + L.scale_off + L.scale_layer * layer) : nullptr;
        a.kmean = fp8 ? (float*)(h->pool + L.mean_off + L.mean_layer * layer) : nullptr;
        a.kpart = !fp8 ? nullptr
                       : static_scratch ? (double*)sptr : (double*)(h->pool + L.part_off + L.part_layer * layer);
        a.table = h->table;
        a.htab = (const double2*)(h->pool + L.htab64_off);
        a.wtab = (const double2*)(h->pool + L.wtab64_off);
        a.omega_t = (const double*)(h->pool + L.omega_off);
        a.N = L.N; a.heads = c.heads; a.D = c.head_dim; a.pt = c.page_tokens; a.ppc = L.ppc;
        a.T = L.T; a.S = c.S;
        a.frame_h = c.frame_h; a.frame_w = c.frame_w;
        a.dt = c.rope_split[0]; a.dh = c.rope_split[1]; a.dw = c.rope_split[2];
        a.slot_first = slot_first; a.nslots = nslots;
        a.in_fp32 = c.in_dtype == WF_DTYPE_FP32;
        a.nblk = L.nblk;
        const hipError_t e = wf::launch_publish(a, fp8, (hipStream_t)stream);
        if (e != hipSuccess) return h->fail_hip(e, "wf_kv_publish launch");
    }
    for (int i = 0; i < nslots; ++i) h->ready[layer] |= 1ull << h->position_of_slot(slot_first + i);
    return WF_OK;
}

int wf_kv_publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                  const void* q, const void* k, const void* v, int64_t row_stride_elems,
                  const int32_t* chunk_t0_host, void* q_out, float* q_scales, void* stream) {
    return publish(h, layer, slot_first, nslots, q, k, v, row_stride_elems, chunk_t0_host, q_out, q_scales,
                   stream, false);
}

int wf_kv_publish_noalloc(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                          const void* q, const void* k, const void* v, int64_t row_stride_elems,
                          const int32_t* chunk_t0_host, void* q_out, float* q_scales, void* stream) {
    return publish(h, layer, slot_first, nslots, q, k, v, row_stride_elems, chunk_t0_host, q_out, q_scales,
                   stream, true);
}

// The fused projection + publish, bf16 operands or (f8) e4m3 codes with
// per-row scales xs / ws.
static int project_publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots, const void* x,
                           int64_t x_row_stride_elems, const float* xs, int32_t hidden, const void* w,
                           const float* ws, const void* bias, const int32_t* chunk_t0_host, void* q_out,
                           void* stream, bool f8) {
    if (!h) return WF_E_INVALID_ARG;
    const wf_config& c = h->cfg;
    const Layout& L = h->L;
    const int esz = f8 ? 1 : 2;                    // bytes per operand element
    const int kstage = 128 / esz;                  // hidden channels per 128-byte stage
    if (layer < 0 || layer >= c.num_layers) return WF_E_INVALID_ARG;
    if (nslots < 1 || slot_first < 0 || slot_first + nslots > c.S + 1) return WF_E_INVALID_ARG;
    if (!x || !w || !q_out) return WF_E_INVALID_ARG;
    if (f8 && (!xs || !ws)) return WF_E_INVALID_ARG;
    if (hidden < kstage || hidden % kstage != 0 || x_row_stride_elems < hidden) return WF_E_INVALID_ARG;
    if (((uintptr_t)x | (uintptr_t)w | (uintptr_t)q_out) % 16 || (x_row_stride_elems * esz) % 16 ||
        ((uintptr_t)bias % 16) || ((uintptr_t)xs % 16) || ((uintptr_t)ws % 16))
        return WF_E_INVALID_ARG;
    const int hd = c.heads * c.head_dim;
    if (c.qk_dtype != WF_DTYPE_BF16 || hd % 128 != 0) return WF_E_SHAPE;
    if (wf::proj_frames_per_tile(c.frame_h * c.frame_w) > wf::kProjMaxFrames) return WF_E_SHAPE;
    if (c.frame_h * (c.rope_split[1] / 2) + c.frame_w * (c.rope_split[2] / 2) > wf::kProjMaxRopeEntries)
        return WF_E_SHAPE;
    const int64_t xbytes = (((int64_t)nslots * L.N - 1) * x_row_stride_elems + hidden) * esz;
    const int64_t wbytes = (int64_t)3 * hd * hidden * esz;
    if (xbytes >= ((int64_t)1 << 31) || wbytes >= ((int64_t)1 << 31)) return WF_E_SHAPE;
    for (int i = 0; i < nslots; ++i)
        if (!h->present(h->position_of_slot(slot_first + i))) {
            snprintf(h->err, sizeof h->err, "slot %d holds no chunk in round %lld", slot_first + i,
                     (long long)h->round());
            return WF_E_INVALID_ARG;
        }
    wf::ProjArgs a{};
    for (int i = 0; i < nslots; ++i) {
        const int64_t t0 = chunk_t0_host
                               ? (int64_t)chunk_t0_host[i]
                               : (int64_t)c.chunk_frames * h->chunk_at(h->position_of_slot(slot_first + i));
        if (t0 < 0 || t0 > INT32_MAX / 2) return WF_E_INVALID_ARG;
        a.t0[i] = (int)t0;
    }
    // live slots take their chunk id from the device round counter (the same
    // values in eager use; right in every round a captured launch replays)
    if (!chunk_t0_host && slot_first + nslots <= c.S + 1) {
        a.ring = h->ring_dev();
        a.t0_round = c.first_round - slot_first;
        a.chunk_frames = c.chunk_frames;
    }
    if (!h->host_model) {
        a.x = x;
        a.x_stride = x_row_stride_elems;
        a.xbytes = (int32_t)xbytes;
        a.w = w;
        a.wbytes = (int32_t)wbytes;
        a.xs = xs;
        a.ws = ws;
        a.bias = (const uint16_t*)bias;
        a.q_out = q_out;
        a.kpage = h->pool + L.k_off + L.k_layer * layer;
        a.vpage = (uint16_t*)(h->pool + L.v_off + L.v_layer * layer);
        a.table = h->table;
        a.htab = (const float2*)(h->pool + L.htab_off);
        a.wtab = (const float2*)(h->pool + L.wtab_off);
        a.omega_t = (const double*)(h->pool + L.omega_off);
        a.N = L.N; a.heads = c.heads; a.D = c.head_dim; a.pt = c.page_tokens; a.ppc = L.ppc;
        a.T = L.T; a.hidden = hidden;
        a.frame_h = c.frame_h; a.frame_w = c.frame_w;
        a.dt = c.rope_split[0]; a.dh = c.rope_split[1]; a.dw = c.rope_split[2];
        a.slot_first = slot_first; a.nslots = nslots;
        a.mtiles = (L.N + wf::kProjTokens - 1) / wf::kProjTokens;
        a.ctiles = (3 * hd + wf::kProjChannels - 1) / wf::kProjChannels;
        a.mrows = nslots * a.mtiles;
        // each XCD takes one block of (channel-tile group x token-row group), so
        // its L2 holds a slice of w and the x rows it is working on
        a.g_ct = a.ctiles >= 4 ? 4 : (a.ctiles >= 2 ? 2 : 1);
        a.g_mt = wf::kXcds / a.g_ct;
        int per = 0;
        for (int xc = 0; xc < wf::kXcds; ++xc) {
            const int cg = xc % a.g_ct, mg = xc / a.g_ct;
            const int nc = (cg + 1) * a.ctiles / a.g_ct - cg * a.ctiles / a.g_ct;
            const int nr = (mg + 1) * a.mrows / a.g_mt - mg * a.mrows / a.g_mt;
            per = std::max(per, nc * nr);
        }
        const hipError_t e = wf::launch_project(a, f8, per * wf::kXcds, (hipStream_t)stream);
        if (e != hipSuccess)
            return h->fail_hip(e, f8 ? "wf_qkv_project_publish_w8a8 launch" : "wf_qkv_project_publish launch");
    }
    for (int i = 0; i < nslots; ++i) h->ready[layer] |= 1ull << h->position_of_slot(slot_first + i);
    return WF_OK;
}

int wf_qkv_project_publish(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                           const void* x, int64_t x_row_stride_elems, int32_t hidden, const void* w,
                           const void* bias, const int32_t* chunk_t0_host, void* q_out, void* stream) {
    return project_publish(h, layer, slot_first, nslots, x, x_row_stride_elems, nullptr, hidden, w, nullptr,
                           bias, chunk_t0_host, q_out, stream, false);
}

int wf_qkv_project_publish_w8a8(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                                const void* x8, int64_t x_row_stride, const float* x_scales, int32_t hidden,
                                const void* w8, const float* w_scales, const void* bias,
                                const int32_t* chunk_t0_host, void* q_out, void* stream) {
    return project_publish(h, layer, slot_first, nslots, x8, x_row_stride, x_scales, hidden, w8, w_scales,
                           bias, chunk_t0_host, q_out, stream, true);
}

int wf_quantize_rows_fp8(const void* x, int64_t rows, int32_t cols, int64_t x_row_stride_elems,
                         uint8_t* codes, int64_t code_row_stride, float* scales, void* stream) {
    if (rows < 0 || !x || !codes || !scales) return WF_E_INVALID_ARG;
    if (cols < 8 || cols % 8 != 0 || cols > wf::kQuantMaxCols) return WF_E_SHAPE;
    if (x_row_stride_elems < cols || x_row_stride_elems % 8 != 0 || code_row_stride < cols ||
        code_row_stride % 8 != 0)
        return WF_E_INVALID_ARG;
    if ((uintptr_t)x % 16 || (uintptr_t)codes % 8 || (uintptr_t)scales % 4) return WF_E_INVALID_ARG;
    if (rows > INT32_MAX) return WF_E_SHAPE;
    if (rows == 0) return WF_OK;
    const hipError_t e = wf::launch_quant_rows((const uint16_t*)x, rows, cols, x_row_stride_elems, codes,
                                               code_row_stride, scales, (hipStream_t)stream);
    return e == hipSuccess ? WF_OK : WF_E_HIP;
}

int wf_attention_round(wf_handle* h, int32_t layer, int32_t slot_first, int32_t nslots,
                       const void* q, const float* q_scales, void* out, int32_t out_dtype,
                       void* stream) {
    if (!h) return WF_E_INVALID_ARG;
    const wf_config& c = h->cfg;
    const Layout& L = h->L;
    if (layer < 0 || layer >= c.num_layers) return WF_E_INVALID_ARG;
    if (nslots < 1 || slot_first < 0 || slot_first + nslots > c.S + 1) return WF_E_INVALID_ARG;
    if (!q || !out) return WF_E_INVALID_ARG;
    if (out_dtype != WF_DTYPE_BF16 && out_dtype != WF_DTYPE_FP32) return WF_E_INVALID_ARG;
    const bool fp8 = c.qk_dtype == WF_DTYPE_FP8_E4M3;
    if (fp8 && !q_scales) return WF_E_INVALID_ARG;
    if (((uintptr_t)q % 16) || ((uintptr_t)out % 16)) return WF_E_INVALID_ARG;
    for (int s = slot_first; s < slot_first + nslots; ++s)
        if (!h->present(h->position_of_slot(s))) {
            snprintf(h->err, sizeof h->err, "slot %d holds no chunk in round %lld", s, (long long)h->round());
            return WF_E_INVALID_ARG;
        }
    // The positions that hold a chunk form at most two runs: the anchors
    // stored so far, [0, anc), and [p2, T - s_lo), from the first occupied
    // non-anchor position to the noisiest occupied slot s_lo (every position
    // in steady rounds: anc = A, p2 = A, s_lo = 0).
    int anc = 0;
    while (anc < h->A() && h->present(anc)) ++anc;
    int p2 = h->A();
    while (p2 < L.T && !h->present(p2)) ++p2;
    int s_lo = 0;
    while (s_lo <= c.S && !h->present(h->position_of_slot(s_lo))) ++s_lo;
    for (int p = 0; p < L.T; ++p) {
        const bool in_runs = p < anc || (p >= p2 && p < L.T - s_lo);
        if (in_runs != h->present(p)) {
            snprintf(h->err, sizeof h->err, "round %lld: occupied positions are not two runs",
                     (long long)h->round());
            return WF_E_SHAPE;
        }
    }
    // readiness check made just before attention: the union of the requested
    // slots' legal contexts is the prefix [0, T - slot_first) (the whole
    // context with the all-live mask), less the positions without a chunk
    const bool all_live = c.live_mask == WF_MASK_ALL_LIVE;
    uint64_t need = h->prefix_bits(all_live ? L.T - s_lo : L.T - slot_first);
    for (int p = 0; p < L.T; ++p)
        if (!h->present(p)) need &= ~(1ull << p);
    if ((h->ready[layer] & need) != need) {
        snprintf(h->err, sizeof h->err, "layer %d: positions 0x%llx not published", layer,
                 (unsigned long long)(need & ~h->ready[layer]));
        return WF_E_NOT_READY;
    }
    if (h->host_model) return WF_OK;
    wf::AttnArgs a{};
    a.q = q; a.q_scales = q_scales; a.out = out;
    a.kpage = h->pool + L.k_off + L.k_layer * layer;
    a.vpage = (const uint16_t*)(h->pool + L.v_off + L.v_layer * layer);
    a.kbytes = (int32_t)L.k_layer;
    a.vbytes = (int32_t)L.v_layer;
    a.kscale = fp8 ? (const float*)(h->pool + L.scale_off + L.scale_layer * layer) : nullptr;
    a.kmean = fp8 ? (const float*)(h->pool + L.mean_off + L.mean_layer * layer) : nullptr;
    a.table = h->table;
    const int wl = slot_first * (c.S + 1) + nslots - 1;
    a.work = (const int32_t*)(h->pool + L.work_off + L.work_stride * wl);
    a.nwork = h->work_count[wl];
    a.N = L.N; a.heads = c.heads; a.D = c.head_dim; a.pt = c.page_tokens; a.ppc = L.ppc;
    a.T = L.T; a.S = c.S;
    a.slot_first = slot_first; a.nslots = nslots;
    a.out_fp32 = out_dtype == WF_DTYPE_FP32;
    a.nblk = L.nblk;
    a.all_live = all_live ? 1 : 0;
    a.anc = anc;
    a.p2 = p2;
    a.end_all = L.T - s_lo;
    a.scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
    const hipError_t e = wf::launch_attention(a, fp8, (hipStream_t)stream);
    if (e != hipSuccess) return h->fail_hip(e, "wf_attention_round launch");
    return WF_OK;
}

// Host side of an advance: one more round, readiness as the advance leaves
// it (anchor kept, history one cleaner, the store's chunk the newest history
// or its anchor, live slots cleared, empty positions unready).
static void advance_host(wf_handle* h) {
    const int A = h->A(), H = h->H();
    const int store = A + H;
    const int store_anchor = h->store_anchor_at_round(h->round());
    h->ring += 1;
    for (int l = 0; l < h->cfg.num_layers; ++l) {
        const uint64_t old = h->ready[l];
        uint64_t nw = old & h->prefix_bits(A);                       // anchor stays
        for (int p = A; p < A + H; ++p)                              // history <- one cleaner
            nw |= ((old >> (p + 1)) & 1ull) << p;
        if (store_anchor >= 0) {                                     // a stored anchor chunk
            nw |= ((old >> store) & 1ull) << store_anchor;
            if (H > 0) nw &= ~(1ull << (A + H - 1));
        }
        for (int p = 0; p < h->L.T; ++p)                             // empty positions stay unready
            if (!h->present(p)) nw &= ~(1ull << p);
        h->ready[l] = nw;                                            // live slots cleared
    }
}

static int check_not_last(wf_handle* h) {
    const int64_t k = h->round();
    if (h->cfg.total_chunks > 0 && k + 1 > (int64_t)h->cfg.total_chunks - 1 + h->S()) {
        snprintf(h->err, sizeof h->err, "round %lld is the last of a %d-chunk video", (long long)k,
                 h->cfg.total_chunks);
        return WF_E_INVALID_ARG;
    }
    return WF_OK;
}

static int check_steady(wf_handle* h) {
    const int64_t k = h->round();
    if (!h->steady_at_round(k) || !h->steady_at_round(k + 1)) {
        snprintf(h->err, sizeof h->err, "round %lld: only steady rounds (every position held, no anchor "
                 "stored) can be captured and replayed", (long long)k);
        return WF_E_INVALID_ARG;
    }
    return WF_OK;
}

int wf_round_advance(wf_handle* h, void* stream) {
    if (!h) return WF_E_INVALID_ARG;
    const int A = h->A(), H = h->H();
    const int store = A + H;
    const int64_t k = h->round();
    int st = check_not_last(h);
    if (st != WF_OK) return st;
    if (h->present(store))
        for (int l = 0; l < h->cfg.num_layers; ++l)
            if (!(h->ready[l] >> store & 1)) {
                snprintf(h->err, sizeof h->err, "layer %d: store not published", l);
                return WF_E_NOT_READY;
            }
    bool capturing = false;
    if (!h->host_model) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        hipError_t e = hipStreamIsCapturing((hipStream_t)stream, &cs);
        if (e != hipSuccess) return h->fail_hip(e, "wf_round_advance capture query");
        capturing = cs == hipStreamCaptureStatusActive;
        if (capturing && (st = check_steady(h)) != WF_OK) return st;
        e = wf::launch_page_table(h->table, h->L.T, A, h->L.ppc, h->ring + 1, h->ring_dev(), store,
                                  h->store_anchor_at_round(k + 1), (hipStream_t)stream);
        if (e != hipSuccess) return h->fail_hip(e, "wf_round_advance launch");
        if (capturing) h->captured = true;
    }
    // a captured advance moves the device counter only when it runs; the host
    // follows each replay through wf_round_replayed
    if (!capturing) advance_host(h);
    return WF_OK;
}

int wf_round_replayed(wf_handle* h) {
    if (!h) return WF_E_INVALID_ARG;
    if (!h->host_model && !h->captured) {
        snprintf(h->err, sizeof h->err, "no advance of this pool was captured: there is no replay to follow");
        return WF_E_INVALID_ARG;
    }
    int st = check_not_last(h);
    if (st == WF_OK) st = check_steady(h);
    if (st != WF_OK) return st;
    // the replayed round published every layer's store (its advance checked
    // that when it was captured)
    const int store = h->A() + h->H();
    for (int l = 0; l < h->cfg.num_layers; ++l) h->ready[l] |= 1ull << store;
    advance_host(h);
    return WF_OK;
}

int wf_round_index(const wf_handle* h, int64_t* k) {
    if (!h || !k) return WF_E_INVALID_ARG;
    *k = h->round();
    return WF_OK;
}

int wf_attention_work_list(const wf_config* cfg, int32_t slot_first, int32_t nslots, int32_t cus_per_xcd,
                           int32_t* units, int64_t capacity, int64_t* count) {
    Layout L{};
    const int st = validate(cfg, &L);
    if (st != WF_OK) return st;
    if (!count || nslots < 1 || slot_first < 0 || slot_first + nslots > cfg->S + 1 || cus_per_xcd < 1)
        return WF_E_INVALID_ARG;
    const std::vector<int32_t> wl = build_work_list(slot_first, nslots, cfg->heads, L.N, L.T,
                                                    cfg->live_mask == WF_MASK_ALL_LIVE,
                                                    cfg->qk_dtype == WF_DTYPE_FP8_E4M3, cus_per_xcd);
    *count = (int64_t)wl.size();
    if (units) {
        if (capacity < (int64_t)wl.size()) return WF_E_INVALID_ARG;
        std::copy(wl.begin(), wl.end(), units);
    }
    return WF_OK;
}

int wf_schedule_chunk_ids(const wf_handle* h, int64_t* ids) {
    if (!h || !ids) return WF_E_INVALID_ARG;
    for (int p = 0; p < h->L.T; ++p) ids[p] = h->present(p) ? h->chunk_at(p) : -1;
    return WF_OK;
}

int wf_page_table_host(const wf_handle* h, int32_t* table) {
    if (!h || !table) return WF_E_INVALID_ARG;
    for (int p = 0; p < h->L.T; ++p)
        for (int i = 0; i < h->L.ppc; ++i) table[p * h->L.ppc + i] = h->group_at(p) * h->L.ppc + i;
    return WF_OK;
}

int wf_ready_mask(const wf_handle* h, int32_t layer, uint64_t* mask) {
    if (!h || !mask || layer < 0 || layer >= h->cfg.num_layers) return WF_E_INVALID_ARG;
    *mask = h->ready[layer];
    return WF_OK;
}

int wf_geometry(const wf_handle* h, int64_t* out) {
    if (!h || !out) return WF_E_INVALID_ARG;
    const Layout& L = h->L;
    const int64_t g[12] = {L.N, L.T, L.ppc, (int64_t)L.k_off, (int64_t)L.v_off, (int64_t)L.k_layer,
                           (int64_t)L.v_layer, (int64_t)L.scale_off, (int64_t)L.scale_layer,
                           (int64_t)L.mean_off, (int64_t)L.mean_layer, L.nblk};
    for (int i = 0; i < 12; ++i) out[i] = g[i];
    return WF_OK;
}

int wf_mfma_calibrate(int32_t blocks, int32_t steps, float* out, void* stream) {
    if (blocks < 1 || steps < 1 || !out) return WF_E_INVALID_ARG;
    const hipError_t e = wf::launch_mfma_calibrate(blocks, steps, out, (hipStream_t)stream);
    return e == hipSuccess ? WF_OK : WF_E_HIP;
}

int wf_stream_copy_calibrate(const void* src, void* dst, int64_t bytes, void* stream) {
    if (!src || !dst || bytes <= 0 || bytes % 16 != 0 || ((uintptr_t)src | (uintptr_t)dst) % 16 != 0)
        return WF_E_INVALID_ARG;
    const hipError_t e = wf::launch_stream_copy(src, dst, bytes, (hipStream_t)stream);
    return e == hipSuccess ? WF_OK : WF_E_HIP;
}

const char* wf_status_string(int status) {
    switch (status) {
        case WF_OK: return "ok";
        case WF_E_INVALID_ARG: return "invalid argument";
        case WF_E_SHAPE: return "unsupported shape or undersized buffer";
        case WF_E_NOT_READY: return "context position not published";
        case WF_E_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* wf_last_error(const wf_handle* h) { return h ? h->err : ""; }

}  // extern "C"
