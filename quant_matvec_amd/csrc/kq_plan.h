// kq_plan.h -- host-side work planning shared by the C ABI layer and the
// kernel launcher.  Plain C++ (no HIP types), so the planning and the
// argument checks can be exercised on a machine without a GPU.
//
// Work decomposition.  A workgroup is one 64-lane wave and processes one
// ITEM: 64 consecutive rows of one tensor (lane i owns row r0+i) over a
// contiguous range of `kchunk` super-block columns.  A tensor with
// kparts > 1 is split along the columns; its items write per-row partial
// sums to a workspace, and the last item of a row tile to finish adds the
// partials in column order and writes y.  The plan of a tensor depends only
// on its own (format, rows, cols, ntok), never on the other members of a
// set, so a tensor computes bitwise the same result alone or in a set.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "../../include/kqmv.h"

namespace kq {

constexpr int kTileRows = 64;             // rows per item: one per lane of a wave64
constexpr int kMaxSet = KQ_MAX_SET;

// Bytes one item stages in LDS for one super-block column (64 rows).  Q6_K
// rows are copied as 53 aligned dwords into a 240-byte LDS row (240/16 odd
// keeps 16-byte LDS reads conflict-free).
constexpr int kSlotBytesQ4K = kTileRows * 144;
constexpr int kSlotBytesQ5K = kTileRows * 176;
constexpr int kSlotBytesQ6K = kTileRows * 240;

struct KqDesc {
    const uint8_t* w;
    const float* x;
    float* y;
    int64_t ldx, ldy;
    int64_t row_bytes;
    int32_t rows;
    int32_t nb;         // super-blocks per row
    int32_t fmt;
    int32_t tiles;      // ceil(rows / 64)
    int32_t kparts;     // column splits per row tile
    int32_t kchunk;     // super-blocks per split (the last may be shorter)
    int32_t item_base;  // first workgroup of this tensor in the grid
    int32_t part_base;  // first partial-sum slot (in items) in the workspace
    int32_t tile_base;  // first counter in the workspace
    int32_t pad;
};

struct KqLaunch {
    KqDesc t[kMaxSet];
    float* partials;      // workspace: [items of split tensors][ntok][64]
    uint32_t* counters;   // workspace: one per row tile of split tensors, zero between calls
    int32_t n;
    int32_t ntok;
    int32_t total_items;
    int32_t lds_bytes;
};

struct KqPlanSizes {
    size_t partial_floats;
    size_t counters;
};

int32_t block_bytes(int32_t fmt);

// Split of one tensor: sets kparts and kchunk.  Depends on (fmt, rows, cols,
// ntok) only.
void plan_tensor(int32_t fmt, int64_t rows, int64_t cols, int32_t ntok,
                 int32_t* kparts, int32_t* kchunk);

// Checks (no HIP calls) of a set; KQ_OK or a KQ_ERR_* code.
int validate_set(const kq_tensor* t, int32_t n, int32_t ntok);

// Fills `out` (workspace pointers left null) and the workspace sizes.
// Assumes validate_set passed.
int build_launch(const kq_tensor* t, int32_t n, int32_t ntok, KqLaunch* out, KqPlanSizes* sizes);

}  // namespace kq
