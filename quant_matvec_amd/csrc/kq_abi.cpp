// kq_abi.cpp -- the extern "C" boundary of libkqmv.so (declared in
// include/kqmv.h): argument checks, work planning, per-stream workspaces
// and the calls into the kernel launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "kq_plan.h"

namespace kq {

int launch_matvec(const KqLaunch& L, hipStream_t stream);
int launch_capacity(const KqLaunch& L);
int plan_pipelined(KqLaunch* L);
void set_pipeline(int mode);
int launch_zero(uint32_t* p, int64_t n, hipStream_t stream);
int scratch_workspace(hipStream_t stream, size_t floats, size_t counters, float** partials, uint32_t** ctrs);
int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream);
int launch_unpack(int32_t fmt, const void* w, int64_t nblocks, int32_t* codes, int32_t* scales,
                  int32_t* mins, float* d, float* dmin, hipStream_t stream);
int launch_dequant(int32_t fmt, const void* w, int64_t rows, int32_t nb, float* out, int64_t ldw,
                   hipStream_t stream);
int launch_embed(const uint8_t* table, int64_t rows, int64_t cols, const int32_t* ids, int32_t n, float* out,
                 int64_t ldo, hipStream_t stream);
int launch_matvec16(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
                    int64_t ldy, int32_t ntok, hipStream_t stream);
int launch_matmul(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
                  int64_t ldy, int32_t ntok, hipStream_t stream);

int32_t block_bytes(int32_t fmt) {
    switch (fmt) {
    case KQ_Q4_K: return 144;
    case KQ_Q5_K: return 176;
    case KQ_Q6_K: return 210;
    default: return KQ_ERR_FORMAT;
    }
}

// LDS of one workgroup: the weight slot of one step (a super-block column
// of a 64-row tile, or the two columns of a segment of a 32-row tile) plus
// one KB of x per token plane and column.
int32_t slot_bytes(int32_t fmt, int32_t ntok, int32_t tile_rows) {
    const bool pair = tile_rows == 32;
    const int32_t w = fmt == KQ_Q4_K ? kSlotBytesQ4K : fmt == KQ_Q5_K ? kSlotBytesQ5K
                    : pair ? kSlotBytesQ6KPair : kSlotBytesQ6K;
    return w + 1024 * ntok * (pair ? 2 : 1);
}

// Tile rows and segment length S.  A matrix with an even number of blocks
// a row runs in 32-row tiles at one token plane (and at two up to kSmallRows
// rows) with two-block segments: two lanes a row, one segment a step, which
// keeps the L2 lines shared by consecutive block columns of a row live for
// only one step per wave, and lets the pipelined kernel take every decode
// set and large matrix.  Otherwise 64-row tiles, one lane a row, with S = 1
// for a matrix of at most kTinyRows rows (few segments a launch: one-block
// runs keep its latency down) and for a Q6_K matrix of at most kSmallRows
// rows with an odd number of blocks a row, else S = 2.  Both tile heights sum
// two-block segments the same way, so where S is 2 at two token counts a
// plane's result does not depend on the height.  Depends only on the
// tensor's own (fmt, rows, cols) and ntok, never on the rest of a set.
constexpr int64_t kSmallRows = 16384;
constexpr int64_t kTinyRows = 1024;
void plan_tensor(int32_t fmt, int64_t rows, int64_t cols, int32_t ntok, int32_t* nseg, int32_t* seg,
                 int32_t* tile_rows) {
    const int64_t nb = cols / 256;
    const bool pair = nb % 2 == 0 && (ntok == 1 || (ntok == 2 && rows <= kSmallRows));
    *tile_rows = pair ? 32 : kTileRows;
    const int32_t S = pair ? 2 : ((fmt == KQ_Q6_K && rows <= kSmallRows && nb % 2) || rows <= kTinyRows) ? 1 : 2;
    *seg = S;
    *nseg = (int32_t)((nb + S - 1) / S);
}

static bool ranges_overlap(uintptr_t a0, uintptr_t a1, uintptr_t b0, uintptr_t b1) {
    return a0 < b1 && b0 < a1;
}

static int validate_tensors(const kq_tensor* t, int32_t n, int32_t ntok, int32_t max_ntok) {
    if (n < 1 || n > kMaxSet) return KQ_ERR_SET_SIZE;
    if (t == nullptr) return KQ_ERR_NULL;
    if (ntok < 1 || ntok > max_ntok) return KQ_ERR_NTOK;
    int64_t items = 0;
    for (int i = 0; i < n; ++i) {
        const kq_tensor& T = t[i];
        if (block_bytes(T.fmt) < 0) return KQ_ERR_FORMAT;
        if (T.cols <= 0 || T.cols % 256) return KQ_ERR_COLS;
        if (T.rows <= 0) return KQ_ERR_ROWS;
        if (!T.w || !T.x || !T.y) return KQ_ERR_NULL;
        if (T.reserved != 0) return KQ_ERR_FORMAT;
        if ((reinterpret_cast<uintptr_t>(T.w) & 15) || (reinterpret_cast<uintptr_t>(T.x) & 15) ||
            (reinterpret_cast<uintptr_t>(T.y) & 3))
            return KQ_ERR_ALIGN;
        if (T.ldx < T.cols || (T.ldx & 3) || T.ldy < T.rows) return KQ_ERR_STRIDE;
        // 32-bit index space of the kernels: a 64-row tile must span < 2^31
        // bytes, rows and per-plane offsets must fit in int32.
        const int64_t rb = (T.cols / 256) * block_bytes(T.fmt);
        if (T.rows > INT32_MAX || rb * kTileRows >= ((int64_t)1 << 31) || T.ldx > ((int64_t)1 << 40) ||
            T.ldy > ((int64_t)1 << 40))
            return KQ_ERR_TOO_LARGE;
        int32_t ns, sg, tr;
        plan_tensor(T.fmt, T.rows, T.cols, ntok, &ns, &sg, &tr);
        items += ((T.rows + tr - 1) / tr) * ns;
        if (items > INT32_MAX / 2) return KQ_ERR_TOO_LARGE;
    }
    // outputs must not overlap each other or any input (hull of the strided ranges)
    for (int i = 0; i < n; ++i) {
        const kq_tensor& A = t[i];
        const uintptr_t y0 = reinterpret_cast<uintptr_t>(A.y);
        const uintptr_t y1 = y0 + (uintptr_t)(((int64_t)(ntok - 1) * A.ldy + A.rows) * 4);
        for (int j = 0; j < n; ++j) {
            const kq_tensor& B = t[j];
            const uintptr_t w0 = reinterpret_cast<uintptr_t>(B.w);
            const uintptr_t w1 = w0 + (uintptr_t)(B.rows * (B.cols / 256) * block_bytes(B.fmt));
            const uintptr_t x0 = reinterpret_cast<uintptr_t>(B.x);
            const uintptr_t x1 = x0 + (uintptr_t)(((int64_t)(ntok - 1) * B.ldx + B.cols) * 4);
            if (ranges_overlap(y0, y1, w0, w1) || ranges_overlap(y0, y1, x0, x1)) return KQ_ERR_OVERLAP;
            if (j != i) {
                const uintptr_t z0 = reinterpret_cast<uintptr_t>(B.y);
                const uintptr_t z1 = z0 + (uintptr_t)(((int64_t)(ntok - 1) * B.ldy + B.rows) * 4);
                if (ranges_overlap(y0, y1, z0, z1)) return KQ_ERR_OVERLAP;
            }
        }
    }
    return KQ_OK;
}

int validate_set(const kq_tensor* t, int32_t n, int32_t ntok) { return validate_tensors(t, n, ntok, KQ_MAX_NTOK); }

int build_launch(const kq_tensor* t, int32_t n, int32_t ntok, int32_t groups, KqLaunch* L) {
    *L = KqLaunch{};
    const int32_t planes = ntok / groups;
    L->h.n = n * groups;
    for (int i = 0; i < kMaxSet; ++i) L->h.wg_end[i] = INT32_MAX;
    L->ntok = planes;
    int32_t lds = 0, segs = 0;
    for (int i = 0; i < n; ++i) {
        const kq_tensor& T = t[i];
        for (int g = 0; g < groups; ++g) {
            KqDesc& D = L->t[i * groups + g];
            D.w = static_cast<const uint8_t*>(T.w);
            D.x = T.x + (int64_t)g * planes * T.ldx;
            D.y = T.y + (int64_t)g * planes * T.ldy;
            D.ldx = T.ldx;
            D.ldy = T.ldy;
            D.nb = (int32_t)(T.cols / 256);
            D.row_bytes = (int64_t)D.nb * block_bytes(T.fmt);
            D.rows = (int32_t)T.rows;
            D.fmt = T.fmt;
            plan_tensor(T.fmt, T.rows, T.cols, ntok, &D.nseg, &D.seg, &D.tile_rows);
            D.tiles = (int32_t)((T.rows + D.tile_rows - 1) / D.tile_rows);
            segs += D.tiles * D.nseg;
            if (slot_bytes(T.fmt, planes, D.tile_rows) > lds) lds = slot_bytes(T.fmt, planes, D.tile_rows);
        }
    }
    L->total_segments = segs;
    L->lds_bytes = lds;
    return KQ_OK;
}

// Token-plane groups.  At ntok >= 3 every tensor runs in 64-row tiles in
// the one-wave kernel, and a wave's compute grows with ntok while its loads
// do not: a launch with few segments (the K/V pair: 208 segments at any
// ntok) leaves most SIMDs idle and waits on a few long waves, and the
// instances for 3 or more planes read x from LDS without the prefetch that
// those for 1 and 2 planes have.  Such a launch splits every tensor's planes
// into G groups of ntok / G, each a member of the same launch planned as at
// the full ntok, so that G times as many workgroups share the compute; each
// group re-reads the weights (from the caches at these sizes).  A plane's
// sums are formed in the same order in every NTOK instance of the kernel,
// so the bits do not depend on G.  With "fits" meaning that the launch's
// segments, G times over, fit one round of resident workgroups (and n * G
// <= kMaxSet), G is
//   * the smallest divisor of ntok that fits with at most 2 planes a group;
//   * else the largest divisor that fits;
//   * else 2 at ntok = 8 for at most kGroupReadBytes of weights (the
//     8-plane instance is the slowest per plane: a decode set of 16
//     rotating layers 59 -> 39 us, a Q6_K FFN down 155 -> 86 us, while the
//     Q4_K FFN matrices lose 3-4% to the second read, and the 202,048-row
//     LM head, whose second read comes from HBM, 20%);
//   * else 1.
// Measured (us per launch, K/V pair at ntok 4 / 6 / 8): 12.7 / 16.7 / 27.4
// with G = 1, 11.9 / 12.1 / 12.5 as chosen; attention output (832
// segments) at ntok 4 / 6 / 8: 18.7 / 27.0 / 31.6 -> 17.1 / 19.7 / 21.8.
constexpr int64_t kGroupReadBytes = (int64_t)128 << 20;
static int g_plane_groups = 0;       // 0: chosen as above; else forced where it divides ntok
void set_plane_groups(int g) { g_plane_groups = g < 0 ? 0 : g; }

static int32_t choose_groups(const kq_tensor* t, int32_t n, int32_t ntok) {
    if (g_plane_groups > 0)
        return (ntok % g_plane_groups == 0 && n * g_plane_groups <= kMaxSet) ? g_plane_groups : 1;
    if (ntok < 3) return 1;
    bool fit[KQ_MAX_NTOK + 1] = {};
    for (int32_t G = 2; G <= ntok; ++G) {
        if (ntok % G || n * G > kMaxSet) continue;
        KqLaunch L;
        build_launch(t, n, ntok, G, &L);
        const int cap = launch_capacity(L);
        fit[G] = cap > 0 && L.total_segments <= cap;
    }
    for (int32_t G = 2; G <= ntok; ++G)
        if (fit[G] && ntok / G <= 2) return G;
    for (int32_t G = ntok; G >= 2; --G)
        if (fit[G]) return G;
    int64_t bytes = 0;
    for (int i = 0; i < n; ++i) bytes += t[i].rows * (t[i].cols / 256) * block_bytes(t[i].fmt);
    if (ntok == 8 && n * 2 <= kMaxSet && bytes <= kGroupReadBytes) return 2;
    return 1;
}

int plan_launch(const kq_tensor* t, int32_t n, int32_t ntok, KqLaunch* L) {
    build_launch(t, n, ntok, choose_groups(t, n, ntok), L);
    plan_pipelined(L);
    return KQ_OK;
}

// Workspace slots of a tensor once its split is set: one per tile while
// the runs are shorter than a tile, else one per run boundary (the kernel's
// shared_slot numbers them the same way).
static int64_t shared_slots(const KqDesc& D) {
    if (D.wg_count <= 1) return 0;
    return D.seg_q < D.nseg ? (int64_t)D.tiles : (int64_t)D.wg_count - 1;
}

// Workgroups of the tensors for a bound C on the bytes of one workgroup's
// run: every tensor's runs hold max(1, C / segment bytes) segments.
static int64_t workgroups_for(const KqLaunch& L, int64_t C, int32_t* per_wg) {
    int64_t P = 0;
    for (int i = 0; i < L.h.n; ++i) {
        const KqDesc& D = L.t[i];
        const int64_t segs = (int64_t)D.tiles * D.nseg;
        const int64_t seg_bytes = (int64_t)D.tile_rows * (D.nb < D.seg ? D.nb : D.seg) * block_bytes(D.fmt);
        int64_t k = C / seg_bytes;
        if (k < 1) k = 1;
        if (k > segs) k = segs;
        if (per_wg) per_wg[i] = (int32_t)k;
        P += (segs + k - 1) / k;
    }
    return P;
}

KqPlanSizes assign_workgroups(KqLaunch* L, int32_t capacity) {
    const int n = L->h.n;
    if (capacity < n) capacity = n;
    // smallest C (bytes) whose split fits in `capacity` workgroups: the
    // workgroup count only falls as C grows, and one workgroup per tensor
    // (C = the largest tensor) always fits
    int64_t lo = 0, hi = 0;
    for (int i = 0; i < n; ++i) {
        const KqDesc& D = L->t[i];
        const int64_t bytes = (int64_t)D.rows * D.row_bytes;
        if (bytes > hi) hi = bytes;
    }
    while (lo < hi) {
        const int64_t mid = lo + (hi - lo) / 2;
        if (workgroups_for(*L, mid, nullptr) <= capacity) hi = mid;
        else lo = mid + 1;
    }
    int32_t k[kMaxSet], P[kMaxSet];
    const int64_t used = workgroups_for(*L, hi, k);
    // workgroups left over go to the tensors in proportion to their bytes
    // (more resident waves keep more bytes in flight on a large launch)
    int64_t total = 0;
    for (int i = 0; i < n; ++i) total += (int64_t)L->t[i].rows * L->t[i].row_bytes;
    const int64_t slack = capacity - used;
    for (int i = 0; i < n; ++i) {
        const KqDesc& D = L->t[i];
        const int32_t segs = D.tiles * D.nseg;
        const int64_t bytes = (int64_t)D.rows * D.row_bytes;
        int64_t p = (segs + k[i] - 1) / k[i] + (total > 0 ? (int64_t)((double)slack * (double)bytes / (double)total) : 0);
        P[i] = (int32_t)(p < segs ? p : segs);
    }
    int32_t base = 0;
    int64_t slots = 0;
    KqPlanSizes sz{0, 0};
    for (int i = 0; i < n; ++i) {
        KqDesc& D = L->t[i];
        const int32_t segs = D.tiles * D.nseg;
        D.wg_base = base;
        D.wg_count = P[i];
        D.seg_q = segs / P[i];
        D.seg_r = segs % P[i];
        base += P[i];
        L->h.wg_end[i] = base;
        // shared-tile slots: one a tile while runs are shorter than a tile,
        // else one a run boundary (at most one boundary lies inside a tile)
        D.part_base = (int32_t)slots;
        D.tile_base = (int32_t)slots;
        const int64_t ns = shared_slots(D);
        slots += ns;
        sz.partial_floats += (size_t)ns * D.nseg * L->ntok * kTileRows;
    }
    L->grid = base;
    L->h.grid = base;
    sz.counters = (size_t)slots;
    return sz;
}

void bind_workspace(KqLaunch* L, float* partials, uint32_t* counters) {
    L->partials = partials;
    L->counters = counters;
    size_t off = 0;
    for (int i = 0; i < L->h.n; ++i) {
        KqDesc& D = L->t[i];
        const int64_t ns = shared_slots(D);
        const bool any = ns > 0 && partials != nullptr;
        D.partials = any ? partials + off : nullptr;
        D.counters = any ? counters + D.tile_base : nullptr;
        off += (size_t)ns * D.nseg * L->ntok * kTileRows;
    }
}

// -------------------------------------------------------------- workspaces
// One per (device, stream): the shared-tile slots and arrival counters of
// the fix-up.  Allocated by the first call on that stream that needs one,
// with room for kWorkspaceFloats slot floats and kWorkspaceCounters counters
// (the slots are bounded by the grid and the row length, so every plan of
// the layer shapes at any ntok fits), its counters zeroed by a fill kernel on
// the stream; every launch leaves the counters it used at zero.  A later
// plan that needs more gets a new, larger workspace the same way, and the
// old one stays allocated (kernels already queued on the stream may still
// use it): no call synchronizes or frees.  kq_release_workspace frees a
// stream's workspaces once the caller has synchronized it.
constexpr size_t kWorkspaceFloats = (size_t)16 << 20;     // 64 MB of slot floats
constexpr size_t kWorkspaceCounters = (size_t)1 << 16;
struct Workspace {
    float* partials = nullptr;
    size_t partial_cap = 0;
    uint32_t* counters = nullptr;
    size_t counter_cap = 0;
    std::vector<void*> retired;
};

static std::mutex g_ws_mutex;
static std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

static int get_workspace(hipStream_t stream, const KqPlanSizes& sz, float** partials, uint32_t** counters) {
    *partials = nullptr;
    *counters = nullptr;
    if (sz.partial_floats == 0 && sz.counters == 0) return KQ_OK;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    Workspace& ws = g_ws[std::make_pair(dev, stream)];
    if (ws.partial_cap < sz.partial_floats || ws.counter_cap < sz.counters) {
        const size_t pc = std::max({sz.partial_floats, kWorkspaceFloats, 2 * ws.partial_cap});
        const size_t cc = std::max({sz.counters, kWorkspaceCounters, 2 * ws.counter_cap});
        float* p = nullptr;
        uint32_t* c = nullptr;
        if (hipMalloc(&p, pc * sizeof(float)) != hipSuccess) return KQ_ERR_HIP;
        if (hipMalloc(&c, cc * sizeof(uint32_t)) != hipSuccess) {
            (void)hipFree(p);
            return KQ_ERR_HIP;
        }
        if (launch_zero(c, (int64_t)cc, stream) != KQ_OK) {
            (void)hipFree(p);
            (void)hipFree(c);
            return KQ_ERR_HIP;
        }
        if (ws.partials) ws.retired.push_back(ws.partials);
        if (ws.counters) ws.retired.push_back(ws.counters);
        ws.partials = p;
        ws.counters = c;
        ws.partial_cap = pc;
        ws.counter_cap = cc;
    }
    *partials = ws.partials;
    *counters = ws.counters;
    return KQ_OK;
}

static int release_workspace(hipStream_t stream) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return KQ_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_ws_mutex);
    auto it = g_ws.find(std::make_pair(dev, stream));
    if (it == g_ws.end()) return KQ_OK;
    int rc = KQ_OK;
    Workspace& ws = it->second;
    ws.retired.push_back(ws.partials);
    ws.retired.push_back(ws.counters);
    for (void* p : ws.retired)
        if (p && hipFree(p) != hipSuccess) rc = KQ_ERR_HIP;
    g_ws.erase(it);
    return rc;
}

// Plans and enqueues one launch of the validated set with the stream's
// workspace.
static int enqueue_set(const kq_tensor* tensors, int32_t n, int32_t ntok, hipStream_t s) {
    KqLaunch L;
    plan_launch(tensors, n, ntok, &L);
    const int cap = launch_capacity(L);
    if (cap <= 0) return KQ_ERR_HIP;
    const KqPlanSizes sz = assign_workgroups(&L, cap);
    float* partials = nullptr;
    uint32_t* counters = nullptr;
    const int rc = get_workspace(s, sz, &partials, &counters);
    if (rc != KQ_OK) return rc;
    bind_workspace(&L, partials, counters);
    return launch_matvec(L, s);
}

}  // namespace kq

using namespace kq;

extern "C" {

int32_t kq_block_bytes(int32_t fmt) { return block_bytes(fmt); }

int64_t kq_row_bytes(int32_t fmt, int64_t cols) {
    const int32_t bb = block_bytes(fmt);
    if (bb < 0) return KQ_ERR_FORMAT;
    if (cols <= 0 || cols % 256) return KQ_ERR_COLS;
    return (cols / 256) * bb;
}

int kq_validate_set(const kq_tensor* tensors, int32_t n, int32_t ntok) {
    return validate_set(tensors, n, ntok);
}

int kq_matvec_set(const kq_tensor* tensors, int32_t n, int32_t ntok, void* stream) {
    const int rc = validate_set(tensors, n, ntok);
    if (rc != KQ_OK) return rc;
    return enqueue_set(tensors, n, ntok, static_cast<hipStream_t>(stream));
}

int kq_release_workspace(void* stream) { return release_workspace(static_cast<hipStream_t>(stream)); }

int kq_debug_set_pipeline(int32_t mode) {
    set_pipeline(mode);
    return KQ_OK;
}

int kq_debug_plan_kernel(const kq_tensor* tensors, int32_t n, int32_t ntok) {
    const int rc = validate_set(tensors, n, ntok);
    if (rc != KQ_OK) return rc;
    KqLaunch L;
    plan_launch(tensors, n, ntok, &L);
    return L.pipelined ? 1 : 0;
}

int kq_debug_set_plane_groups(int32_t groups) {
    set_plane_groups(groups);
    return KQ_OK;
}

int kq_debug_plan_plane_groups(const kq_tensor* tensors, int32_t n, int32_t ntok) {
    const int rc = validate_set(tensors, n, ntok);
    if (rc != KQ_OK) return rc;
    KqLaunch L;
    plan_launch(tensors, n, ntok, &L);
    return ntok / L.ntok;
}

int kq_matvec_set_noalloc(const kq_tensor* tensors, int32_t n, int32_t ntok, void* stream) {
    int rc = validate_set(tensors, n, ntok);
    if (rc != KQ_OK) return rc;
    hipStream_t s = static_cast<hipStream_t>(stream);
    KqLaunch L;
    plan_launch(tensors, n, ntok, &L);
    const int cap = launch_capacity(L);
    if (cap <= 0) return KQ_ERR_HIP;
    const KqPlanSizes sz = assign_workgroups(&L, cap);
    float* partials = nullptr;
    uint32_t* counters = nullptr;
    rc = scratch_workspace(s, sz.partial_floats, sz.counters, &partials, &counters);
    if (rc != KQ_OK) return rc;
    bind_workspace(&L, partials, counters);
    return launch_matvec(L, s);
}

int kq_matvec(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx,
              float* y, int64_t ldy, int32_t ntok, void* stream) {
    kq_tensor t;
    t.fmt = fmt;
    t.reserved = 0;
    t.w = w;
    t.x = x;
    t.y = y;
    t.rows = rows;
    t.cols = cols;
    t.ldx = ldx;
    t.ldy = ldy;
    return kq_matvec_set(&t, 1, ntok, stream);
}

int kq_matvec16(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
                int64_t ldy, int32_t ntok, void* stream) {
    kq_tensor t;
    t.fmt = fmt;
    t.reserved = 0;
    t.w = w;
    t.x = x;
    t.y = y;
    t.rows = rows;
    t.cols = cols;
    t.ldx = ldx;
    t.ldy = ldy;
    const int rc = validate_tensors(&t, 1, ntok, KQ_MAX_NTOK16);
    if (rc != KQ_OK) return rc;
    if ((rows + 15) / 16 > INT32_MAX) return KQ_ERR_TOO_LARGE;
    return launch_matvec16(fmt, w, rows, cols, x, ldx, y, ldy, ntok, static_cast<hipStream_t>(stream));
}

int kq_matmul(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
              int64_t ldy, int32_t ntok, void* stream) {
    kq_tensor t;
    t.fmt = fmt;
    t.reserved = 0;
    t.w = w;
    t.x = x;
    t.y = y;
    t.rows = rows;
    t.cols = cols;
    t.ldx = ldx;
    t.ldy = ldy;
    const int rc = validate_tensors(&t, 1, ntok, KQ_MAX_MATMUL_NTOK);
    if (rc != KQ_OK) return rc;
    if ((rows + 15) / 16 > INT32_MAX) return KQ_ERR_TOO_LARGE;
    return launch_matmul(fmt, w, rows, cols, x, ldx, y, ldy, ntok, static_cast<hipStream_t>(stream));
}

int kq_unpack_blocks(int32_t fmt, const void* w, int64_t nblocks, int32_t* codes_out, int32_t* scales_out,
                     int32_t* mins_out, float* d_out, float* dmin_out, void* stream) {
    if (block_bytes(fmt) < 0) return KQ_ERR_FORMAT;
    if (nblocks <= 0) return KQ_ERR_ROWS;
    if (!w) return KQ_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(w) & 15) return KQ_ERR_ALIGN;
    if (nblocks > ((int64_t)1 << 31) * 255) return KQ_ERR_TOO_LARGE;
    return launch_unpack(fmt, w, nblocks, codes_out, scales_out, mins_out, d_out, dmin_out,
                         static_cast<hipStream_t>(stream));
}

int kq_dequant(int32_t fmt, const void* w, int64_t rows, int64_t cols, float* out, int64_t ldw, void* stream) {
    if (block_bytes(fmt) < 0) return KQ_ERR_FORMAT;
    if (cols <= 0 || cols % 256) return KQ_ERR_COLS;
    if (rows <= 0) return KQ_ERR_ROWS;
    if (!w || !out) return KQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(w) & 15) || (reinterpret_cast<uintptr_t>(out) & 3)) return KQ_ERR_ALIGN;
    if (ldw < cols) return KQ_ERR_STRIDE;
    if (rows * (cols / 256) > ((int64_t)1 << 31) * 255) return KQ_ERR_TOO_LARGE;
    return launch_dequant(fmt, w, rows, (int32_t)(cols / 256), out, ldw, static_cast<hipStream_t>(stream));
}

int kq_embed_rows(int32_t fmt, const void* table, int64_t rows, int64_t cols, const int32_t* ids, int32_t n,
                  float* out, int64_t ldo, void* stream) {
    if (fmt != KQ_Q4_K) return KQ_ERR_FORMAT;
    if (cols <= 0 || cols % 256) return KQ_ERR_COLS;
    if (rows <= 0 || n < 1 || n > KQ_MAX_EMBED_IDS) return KQ_ERR_ROWS;
    if (!table || !ids || !out) return KQ_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(table) & 15) || (reinterpret_cast<uintptr_t>(ids) & 3) ||
        (reinterpret_cast<uintptr_t>(out) & 15))
        return KQ_ERR_ALIGN;
    if (ldo < cols || (ldo & 3)) return KQ_ERR_STRIDE;
    const int64_t groups = (cols / 256 + 3) / 4;
    if (rows > INT32_MAX || n * groups > INT32_MAX || ldo > ((int64_t)1 << 40)) return KQ_ERR_TOO_LARGE;
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out);
    const uintptr_t o1 = o0 + (uintptr_t)(((int64_t)(n - 1) * ldo + cols) * 4);
    const uintptr_t t0 = reinterpret_cast<uintptr_t>(table);
    const uintptr_t t1 = t0 + (uintptr_t)(rows * (cols / 256) * 144);
    const uintptr_t i0 = reinterpret_cast<uintptr_t>(ids);
    const uintptr_t i1 = i0 + (uintptr_t)n * 4;
    if (ranges_overlap(o0, o1, t0, t1) || ranges_overlap(o0, o1, i0, i1)) return KQ_ERR_OVERLAP;
    return launch_embed(static_cast<const uint8_t*>(table), rows, cols, ids, n, out, ldo,
                        static_cast<hipStream_t>(stream));
}

int kq_debug_read_probe(const void* buf, int64_t bytes, void* sink, void* stream) {
    if (!buf || !sink) return KQ_ERR_NULL;
    if (bytes <= 0 || (bytes & 15)) return KQ_ERR_ROWS;
    if ((reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3)) return KQ_ERR_ALIGN;
    return launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink), static_cast<hipStream_t>(stream));
}

const char* kq_strerror(int code) {
    switch (code) {
    case KQ_OK: return "ok";
    case KQ_ERR_FORMAT: return "unsupported format (only Q4_K=12, Q5_K=13, Q6_K=14)";
    case KQ_ERR_COLS: return "cols must be a positive multiple of 256";
    case KQ_ERR_ROWS: return "rows (or block count) must be positive";
    case KQ_ERR_NTOK: return "ntok must be in 1..8 (1..16 for kq_matvec16, 1..2^20 for kq_matmul)";
    case KQ_ERR_NULL: return "null pointer";
    case KQ_ERR_ALIGN: return "misaligned pointer (w, x need 16 bytes; y 4 bytes)";
    case KQ_ERR_STRIDE: return "bad leading dimension (ldx >= cols and a multiple of 4; ldy >= rows)";
    case KQ_ERR_OVERLAP: return "an output overlaps another output or an input";
    case KQ_ERR_SET_SIZE: return "set size must be in 1..16";
    case KQ_ERR_HIP: return "HIP runtime error";
    case KQ_ERR_TOO_LARGE: return "size exceeds the kernels' index space";
    case KQ_ERR_SCRATCH:
        return "the plan needs more shared-tile sums than kq_matvec_set_noalloc's fixed scratch holds "
               "(16 MB of sums, 65,536 counters); use kq_matvec_set";
    default: return "unknown status";
    }
}

int kq_version(void) { return KQMV_ABI_VERSION; }

}  // extern "C"
