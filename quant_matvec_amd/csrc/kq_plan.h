// kq_plan.h -- host-side work planning shared by the C ABI layer and the
// kernel launcher.  Plain C++ (no HIP types), so the planning and the
// argument checks can be exercised on a machine without a GPU.
//
// Work decomposition.  Rows are taken 64 at a time (a TILE: one row per
// lane of a wave64).  Each tile row is cut into SEGMENTS of S consecutive
// super-blocks (S = 2, or 1 for a Q6_K matrix of at most 16384 rows and for
// any matrix of at most 1024 rows); the segments of a tensor are numbered
// tile-major.  The row results of a tile are the ordered sum
// ((0 + seg_0) + seg_1) + ... of its segment sums, each segment accumulated
// block by block.  S depends only on the tensor's own shape, so a tensor
// computes bitwise the same result alone or in a set, and whatever
// workgroup does the work.
//
// The launch is a grid of one-wave workgroups, at most one full round of
// resident waves, split between the tensors of the set: tensor i gets P_i
// workgroups, each streaming a contiguous run of its segments (the runs'
// lengths differ by at most one), prefetching ahead across segment and tile
// boundaries.  The P_i are chosen so that the largest run, in weight bytes,
// is as small as the round of resident waves allows.  A tile whose segments
// all belong to one workgroup is summed in registers and written directly;
// a tile shared by workgroups has its segment sums written to a workspace
// slot, and the last contributor (an arrival counter per slot) adds them in
// order.  A shared tile holds a run boundary, and its slot is numbered by
// the first boundary inside it, so a tensor of P workgroups needs at most
// P - 1 slots of nseg * ntok * 64 floats: the workspace is bounded by the
// grid and the row length, not by the number of rows.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/kqmv.h"

namespace kq {

constexpr int kTileRows = 64;             // rows per item: one per lane of a wave64
constexpr int kMaxSet = KQ_MAX_SET;

// Bytes one item stages in LDS for one super-block column (64 rows).  Q6_K
// rows are copied as 52 aligned dwords into a 208-byte LDS row (208/16 odd
// keeps 16-byte LDS reads conflict-free) plus word 52 of each row apart.
constexpr int kSlotBytesQ4K = kTileRows * 144;
constexpr int kSlotBytesQ5K = kTileRows * 176;
constexpr int kSlotBytesQ6K = kTileRows * 208 + 4 * kTileRows;
// 32-row tiles stage the two blocks of a segment per step: Q4_K/Q5_K the
// same bytes as a 64-row column; Q6_K 32 rows of 26 chunks (words 0..103
// of the pair's 105) and word 104 of each row apart (64 words: the direct
// loads of the pipelined kernel write one per lane).
constexpr int kSlotBytesQ6KPair = 32 * 416 + 4 * 64;

struct KqDesc {
    const uint8_t* w;
    const float* x;
    float* y;
    int64_t ldx, ldy;
    int64_t row_bytes;
    int32_t rows;
    int32_t nb;         // super-blocks per row
    int32_t fmt;
    int32_t tiles;      // ceil(rows / tile_rows)
    int32_t nseg;       // segments per tile row
    int32_t seg;        // S: super-blocks per segment (the last one of a row may be shorter)
    int32_t part_base;  // first shared-tile slot of this tensor in the workspace
    int32_t tile_base;  // first counter (one per shared-tile slot) in the workspace
    int32_t wg_base;    // first workgroup of this tensor
    int32_t wg_count;   // P_i: workgroups of this tensor
    int32_t seg_q;      // workgroup u of the tensor streams segments [u*seg_q + min(u, seg_r), ...),
    int32_t seg_r;      //   seg_q + (u < seg_r) of them
    float* partials;    // this tensor's shared-tile slots in the workspace: [P-1][nseg][ntok][64]
    uint32_t* counters; // this tensor's arrival counters: one per slot, zero between calls
    int32_t tile_rows;  // 64, or 32 for a large matrix (two lanes a row, a segment a step)
    int32_t reserved0;  // pipelined kernel: weight slots R | fold slots TS << 8 | non-temporal loads << 16
    int64_t reserved1;
};
static_assert(sizeof(KqDesc) == 128, "descriptor is four 32-byte groups");

// Read by every workgroup before anything else (in one batch).
struct KqHead {
    int32_t n;
    int32_t grid;             // workgroups of the launch (gridDim.x), read with the rest of the head
    int32_t reserved[6];
    int32_t wg_end[kMaxSet];  // t[i].wg_base + t[i].wg_count; INT32_MAX past the last tensor
};
static_assert(sizeof(KqHead) == 96, "head is three 32-byte groups");

struct KqLaunch {
    KqHead h;
    KqDesc t[kMaxSet];
    float* partials;      // workspace base: shared-tile slots of every tensor
    uint32_t* counters;   // workspace base: one counter per slot
    int32_t ntok;
    int32_t grid;         // workgroups
    int32_t lds_bytes;
    int32_t total_segments;
    int32_t pipelined;    // run by the producer/consumer kernel (one workgroup a compute unit)
    int32_t reserved;
};

struct KqPlanSizes {
    size_t partial_floats;
    size_t counters;
};

int32_t block_bytes(int32_t fmt);

// Segment length S (super-blocks) of one tensor, the segments per tile row
// and the rows of a tile (64, or 32).  Depends on (fmt, rows, cols) and, through
// the tile height, on ntok.
void plan_tensor(int32_t fmt, int64_t rows, int64_t cols, int32_t ntok, int32_t* nseg, int32_t* seg,
                 int32_t* tile_rows);

// LDS bytes of one column step of a tensor (weights, then x per token).
int32_t slot_bytes(int32_t fmt, int32_t ntok, int32_t tile_rows);

// Checks (no HIP calls) of a set; KQ_OK or a KQ_ERR_* code.
int validate_set(const kq_tensor* t, int32_t n, int32_t ntok);

// Fills `out` (workspace pointers and the workgroup split left unset) with
// the tensors' token planes in `groups` groups of ntok / groups planes (a
// divisor of ntok, n * groups <= kMaxSet): member i * groups + g is plane
// group g of tensor i, planned as at the full ntok.  Assumes validate_set
// passed.
int build_launch(const kq_tensor* t, int32_t n, int32_t ntok, int32_t groups, KqLaunch* out);

// build_launch with the plane groups chosen for the current device (or set
// by kq_debug_set_plane_groups), then plan_pipelined.
int plan_launch(const kq_tensor* t, int32_t n, int32_t ntok, KqLaunch* out);

// Splits the launch's workgroups between its tensors for at most
// `capacity` workgroups: sets wg_base, wg_count, seg_q, seg_r, part_base
// and tile_base of every tensor, the head's wg_end and the grid, and
// returns the workspace the split needs (shared-tile slots and counters).
KqPlanSizes assign_workgroups(KqLaunch* L, int32_t capacity);

// Points every tensor's partials and counters into a workspace of the size
// assign_workgroups returned (null pointers for a tensor that needs none).
void bind_workspace(KqLaunch* L, float* partials, uint32_t* counters);

}  // namespace kq
