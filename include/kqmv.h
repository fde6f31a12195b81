/*
 * kqmv.h -- C ABI of the k-quant decode matvec library (libkqmv.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes y = W x for weight matrices stored as k-quant
 * super-blocks, dequantizing every weight on the fly inside the kernel and
 * never writing a dequantized weight to memory (muser-book Ch 13 "The QKV +
 * gate matvec family", section 13.1).  Formats and byte layouts are those of
 * muser-book Ch 6 "The kquant family on the reference lane": Q4_K (section
 * 6.2, Figures 6.2-6.3), Q5_K and Q6_K (section 6.4, Figures 6.4-6.5).
 *
 * Conventions shared by every entry point:
 *   - Pointers named w, x, y, *_out are DEVICE pointers (hipMalloc'd memory
 *     or any device-accessible allocation).  kq_tensor arrays are HOST
 *     memory and are copied into the launch, so they may be freed on return.
 *   - The caller owns all device memory.  Work is enqueued on `stream` (a
 *     hipStream_t, NULL = the default stream) and completes asynchronously;
 *     no entry point synchronizes.  Results may be read after the stream is
 *     synchronized.
 *   - Every check runs on the host before any HIP call; a failed check
 *     returns a negative KQ_ERR_* code and enqueues nothing.  A launch
 *     failure reported by the HIP runtime returns KQ_ERR_HIP.  Nothing is
 *     printed and no exception crosses the ABI.
 *   - Weights: a row-major matrix of `rows` rows, each one contiguous run of
 *     cols/256 super-blocks (muser-book Ch 13 section 13.3; Ch 6 section
 *     6.6), i.e. rows * kq_row_bytes(fmt, cols) bytes.  `w` may point into a
 *     larger allocation (a view into a mapped model arena) but must be
 *     16-byte aligned.
 *   - Activations: x is float32 [ntok][ldx], y is float32 [ntok][ldy]
 *     (plane t of x is x + t*ldx; ldx >= cols, ldy >= rows).  x must be
 *     16-byte aligned and ldx a multiple of 4; y must be 4-byte aligned.
 *   - Results are deterministic run to run.  Each output equals the exact
 *     sum of W[i,j]*x[j] within a few float32 rounding steps relative to
 *     sum_j |W[i,j]*x[j]| (each Q4_K/Q5_K weight is formed with one rounding
 *     and then multiplied in; Q6_K signed codes are multiplied in and their
 *     sub-block sum scaled once; sums accumulate in float32 in a fixed
 *     order), so they are not bitwise equal to another kernel's.
 *   - Up to 16 devices; calls on one device that run concurrently on
 *     different streams are safe.  kq_matvec and kq_matvec_set split long
 *     rows between workgroups; the partial sums of the tiles they share go
 *     to a workspace owned by the library, one per (device, stream).  It is
 *     allocated (hipMalloc, 64 MB of partial sums) by the first call on that
 *     stream that needs one -- make that call outside HIP graph capture --
 *     and is large enough for every plan of a model layer's shapes, since
 *     the partial sums needed are bounded by the grid and the row length,
 *     not by the number of rows.  A later plan that needs more gets a larger
 *     workspace without synchronizing: the old one is kept, never freed
 *     while work may use it.  No entry point synchronizes or frees.
 *     kq_release_workspace frees a stream's workspaces.
 */
#ifndef KQMV_H
#define KQMV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* GGUF tensor type ids (muser-book Ch 6 section 6.1, the GgmlType list). */
enum kq_format { KQ_Q4_K = 12, KQ_Q5_K = 13, KQ_Q6_K = 14 };

enum kq_status {
    KQ_OK = 0,
    KQ_ERR_FORMAT = -1,    /* format is not Q4_K, Q5_K or Q6_K (refused, never converted) */
    KQ_ERR_COLS = -2,      /* cols <= 0 or not a multiple of 256 */
    KQ_ERR_ROWS = -3,      /* rows <= 0 */
    KQ_ERR_NTOK = -4,      /* ntok outside 1..8 */
    KQ_ERR_NULL = -5,      /* a required pointer is NULL */
    KQ_ERR_ALIGN = -6,     /* w or x not 16-byte aligned, y not 4-byte aligned */
    KQ_ERR_STRIDE = -7,    /* ldx < cols, ldx not a multiple of 4, or ldy < rows */
    KQ_ERR_OVERLAP = -8,   /* an output range overlaps another output or an input */
    KQ_ERR_SET_SIZE = -9,  /* n outside 1..KQ_MAX_SET */
    KQ_ERR_HIP = -10,      /* the HIP runtime reported an error */
    KQ_ERR_TOO_LARGE = -11, /* a size exceeds the kernels' 32-bit index space */
    KQ_ERR_SCRATCH = -12    /* kq_matvec_set_noalloc: the plan needs more than its fixed scratch */
};

#define KQ_MAX_SET 16
#define KQ_MAX_NTOK 8
#define KQ_MAX_EMBED_IDS (1 << 24)
#define KQ_MAX_NTOK16 16
#define KQ_MAX_MATMUL_NTOK (1 << 20)

/* One member of a grid-split set. */
typedef struct kq_tensor {
    int32_t fmt;          /* enum kq_format */
    int32_t reserved;     /* must be 0 */
    const void* w;        /* device weights, rows * kq_row_bytes(fmt, cols) bytes */
    const float* x;       /* device activations [ntok][ldx] read by this tensor */
    float* y;             /* device outputs [ntok][ldy] written by this tensor */
    int64_t rows;
    int64_t cols;
    int64_t ldx;
    int64_t ldy;
} kq_tensor;

/* Bytes per 256-weight super-block: 144, 176 or 210 (muser-book Ch 6
 * Figure 6.1); KQ_ERR_FORMAT for any other format. */
int32_t kq_block_bytes(int32_t fmt);

/* Bytes of one row of `cols` weights: cols/256 * kq_block_bytes(fmt)
 * (muser-book Ch 6 section 6.6); a negative KQ_ERR_* code on bad input. */
int64_t kq_row_bytes(int32_t fmt, int64_t cols);

/*
 * y[t][i] = sum_j W[i,j] * x[t][j] for t < ntok and i < rows
 * (muser-book Ch 13 section 13.1; ntok columns as the batch-width rungs of
 * Ch 6 Figure 6.7, served here by one kernel that reads every weight byte
 * once and uses it ntok times).  ntok in 1..8.
 * Returns KQ_OK or a negative KQ_ERR_* code.
 */
int kq_matvec(int32_t fmt, const void* w, int64_t rows, int64_t cols,
              const float* x, int64_t ldx, float* y, int64_t ldy,
              int32_t ntok, void* stream);

/*
 * n independent matvecs in ONE kernel launch (the concurrent Q/K/V/gate set
 * of muser-book Ch 13 section 13.5, issued as one grid the way the
 * opus_gdn_qsa audit's gemv_cat splits its grid between tensors).  Each
 * tensor has its own format, weights, x plane(s) and output; tensors may
 * share x.  Outputs must be pairwise disjoint and must not overlap any
 * weights or activations.  Every workgroup works on one tensor only, so
 * each tensor's result is bitwise equal to a kq_matvec call on it.
 * n in 1..KQ_MAX_SET, ntok in 1..8 (common to the set).
 */
int kq_matvec_set(const kq_tensor* tensors, int32_t n, int32_t ntok, void* stream);

/*
 * kq_matvec_set for callers that cannot allocate: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  Same
 * arguments, checks, results (bitwise equal to kq_matvec_set) and errors,
 * but it allocates nothing, not even on its first call: the partial sums of
 * tiles split between workgroups go to a fixed scratch array in device
 * memory that the library holds on every GPU it runs on until the process
 * ends (16 MB of sums and 65,536 counters).  A plan that needs more returns
 * KQ_ERR_SCRATCH before any HIP call that enqueues work; decode sets of a
 * model layer at ntok 1..8 and the 202,048-row matvec at ntok 1..2 fit.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one
 * GPU (on different streams, or from different threads) race.  The first
 * call on a device enqueues a fill of the scratch's counters on `stream`.
 */
int kq_matvec_set_noalloc(const kq_tensor* tensors, int32_t n, int32_t ntok, void* stream);

/*
 * Frees the workspaces kq_matvec / kq_matvec_set hold for `stream` on the
 * current device (the caller first synchronizes the stream, or destroys it
 * after this call; no queued work may still use them).  The next call on
 * that stream allocates afresh.  Returns KQ_OK, or KQ_ERR_HIP if a free
 * failed.
 */
int kq_release_workspace(void* stream);

/*
 * Host-only validation of a set (the checks kq_matvec_set runs before any
 * HIP call).  Makes no HIP call at all.  Returns KQ_OK or the error code
 * kq_matvec_set would return.
 */
int kq_validate_set(const kq_tensor* tensors, int32_t n, int32_t ntok);

/*
 * The same product as kq_matvec for ntok in 1..KQ_MAX_NTOK16 token planes
 * (up to the 16-token verify width of muser-book Ch 6 section 6.8, whose
 * weight-stationary tile this follows), computed on the matrix cores:
 *   y[t][i] = sum_j W[i,j] x[t][j],  t < ntok.
 * Arguments, layouts, alignment and errors as kq_matvec (w 16-byte aligned,
 * x [ntok][ldx] 16-byte aligned with ldx >= cols a multiple of 4, y
 * [ntok][ldy] 4-byte aligned with ldy >= rows, y disjoint from w and x),
 * except KQ_ERR_NTOK for ntok outside 1..16.  Every weight byte is read
 * once for all planes.  Results meet the same per-row tolerance as
 * kq_matvec but are not bitwise equal to it (another reduction order); a
 * plane's result does not depend on ntok.  Allocates nothing.
 */
int kq_matvec16(int32_t fmt, const void* w, int64_t rows, int64_t cols,
                const float* x, int64_t ldx, float* y, int64_t ldy,
                int32_t ntok, void* stream);

/*
 * The same product for a batch of ntok in 1..KQ_MAX_MATMUL_NTOK token planes
 * (the prefill rung of the batch-width ladder, muser-book Ch 6 Figure 6.7):
 *   y[t][i] = sum_j W[i,j] x[t][j],  t < ntok,
 * on the matrix cores, each block decoded once for 32 tokens.  Arguments,
 * layouts, alignment and errors as kq_matvec16, with ntok up to 2^20.
 * Results meet the same per-row tolerance; a plane's result does not depend
 * on ntok or on the other planes.  Allocates nothing.
 */
int kq_matmul(int32_t fmt, const void* w, int64_t rows, int64_t cols,
              const float* x, int64_t ldx, float* y, int64_t ldy,
              int32_t ntok, void* stream);

/*
 * The embedding lookup of muser-book Ch 6 section 6.7: row ids[t] of a Q4_K
 * table, dequantized, for t < n.
 *   out[t][j] = d*sc_s*q - dmin*m_s of element j of row ids[t]
 * (Ch 6 sections 6.2-6.3; s = sub-block of 32).  Each value is the exact
 * weight correctly rounded to float32 (the products are exact, the
 * difference is rounded once), so a row is bit-equal to kq_dequant of it.
 *   fmt    only KQ_Q4_K: the pages admit a Q4_K (or F16) embedding table and
 *          refuse anything else (Ch 6 section 6.1); other formats return
 *          KQ_ERR_FORMAT.
 *   table  device, rows x cols/256 blocks row-major (cols/256*144 bytes a
 *          row, Ch 6 section 6.6), 16-byte aligned, owned by the caller.
 *   ids    device int32 [n], 4-byte aligned; n in 1..KQ_MAX_EMBED_IDS.  An id
 *          outside [0, rows) gives a row of NaN; nothing outside the table
 *          is read.
 *   out    device float32 [n][ldo], 16-byte aligned, ldo >= cols and a
 *          multiple of 4; must not overlap the table or ids.
 * Enqueued on `stream`; allocates nothing.  All checks run on the host
 * before any HIP call.  Returns KQ_OK or a negative KQ_ERR_* code
 * (KQ_ERR_ROWS for rows or n out of range).
 */
int kq_embed_rows(int32_t fmt, const void* table, int64_t rows, int64_t cols,
                  const int32_t* ids, int32_t n, float* out, int64_t ldo, void* stream);

/*
 * Debug/test export: integer decode of `nblocks` consecutive super-blocks
 * starting at w (16-byte aligned), with the same device decoders the matvec
 * kernels use: the f16 headers, the 6-bit scales and mins of the Q4_K/Q5_K
 * strip (muser-book Ch 6 section 6.2, the get_scale_min rule, Figure 6.3),
 * the 4- and 5-bit codes (Figures 6.2 and 6.4) and the Q6_K int8 scales and
 * 6-bit codes with their -32 offset (section 6.4, Figure 6.5).  Enqueued on
 * `stream`; allocates nothing; all checks on the host (KQ_ERR_FORMAT,
 * KQ_ERR_ROWS for nblocks <= 0, KQ_ERR_NULL for a null w, KQ_ERR_ALIGN).
 * Outputs (device pointers, any may be NULL to skip):
 *   codes_out  int32 [nblocks][256]: Q4_K 0..15, Q5_K 0..31,
 *              Q6_K -32..31 (the 6-bit code minus 32)
 *   scales_out int32 [nblocks][16]: Q4_K/Q5_K sc_0..sc_7 then zeros;
 *              Q6_K the 16 signed int8 sub-block scales
 *   mins_out   int32 [nblocks][16]: Q4_K/Q5_K m_0..m_7 then zeros; Q6_K zeros
 *   d_out, dmin_out float [nblocks]: the f16 headers widened to float
 *              (Q6_K dmin = 0)
 * Returns KQ_OK or a negative KQ_ERR_* code.
 */
int kq_unpack_blocks(int32_t fmt, const void* w, int64_t nblocks,
                     int32_t* codes_out, int32_t* scales_out, int32_t* mins_out,
                     float* d_out, float* dmin_out, void* stream);

/*
 * Debug/test export: dequantized weights as float32 [rows][ldw]
 * (ldw >= cols): Q4_K/Q5_K d*sc_j*q - dmin*m_j, Q6_K d*sc_j*(q - 32) with q
 * the unsigned 6-bit code (muser-book Ch 6 sections 6.2 and 6.4).  Both products are exact in float32 and the
 * difference is rounded once, so each value is the exact weight correctly
 * rounded to float32.  The matvec kernels never call this.
 */
int kq_dequant(int32_t fmt, const void* w, int64_t rows, int64_t cols,
               float* out, int64_t ldw, void* stream);

/*
 * Calibration export, not part of the matvec: one launch of a trivial
 * streaming read over `bytes` bytes at buf (device, 16-byte aligned, bytes a
 * positive multiple of 16), with 16-byte nontemporal loads and nothing else
 * (eight in flight per thread, 32 workgroups of 256 a compute unit), so its rate
 * is what HBM delivers to a kernel on this GPU.  sink: a device uint32 that
 * is written only when a fixed XOR value turns up (callers ignore it).
 * Returns KQ_OK or a negative KQ_ERR_* code (KQ_ERR_ROWS for a bad size).
 */
int kq_debug_read_probe(const void* buf, int64_t bytes, void* sink, void* stream);

/*
 * Debug/test export: which launches of kq_matvec, kq_matvec_set and
 * kq_matvec_set_noalloc may take the pipelined producer/consumer kernel
 * instead of the one-wave-workgroup kernel.  mode = 0: none; mode = 1 (the
 * default, unless the environment sets KQMV_PIPELINE=0): launches whose
 * tensors all run in 32-row tiles at ntok <= 2 and that have at least four
 * segment steps a compute unit; mode = 2: such launches of any size (for
 * tests of small shapes).  Values below 0 act as 0, above 2 as 2.  Both
 * kernels give the same bits.  Process-wide; not for use while other
 * threads launch.  Returns KQ_OK.
 */
int kq_debug_set_pipeline(int32_t mode);

/*
 * Debug/test export: which kernel kq_matvec_set would launch for this set
 * on the current device: 1 the pipelined producer/consumer kernel, 0 the
 * one-wave-workgroup kernel, or a negative KQ_ERR_* code if the set is
 * invalid (the kq_validate_set checks).  Launches nothing; reads only the
 * descriptors (not the buffers they point to).
 */
int kq_debug_plan_kernel(const kq_tensor* tensors, int32_t n, int32_t ntok);

/*
 * Debug/test export: token-plane groups of kq_matvec, kq_matvec_set and
 * kq_matvec_set_noalloc.  A launch at ntok >= 3 with few segments splits
 * each tensor's ntok planes into G groups of ntok / G planes, run as
 * separate members of the one launch with the plan of the full ntok (more
 * workgroups share the compute; each group reads the weights again).
 * groups = 0 (the default): G chosen per launch from the segment count,
 * the resident workgroups of the device and ntok (G = 1 at ntok <= 2).
 * groups >= 1: G = groups wherever it divides ntok and
 * n * groups <= 16, else 1 (for tests).  Negative values act as 0.  Every
 * G gives the same bits.  Process-wide; not for use while other threads
 * launch.  Returns KQ_OK.
 */
int kq_debug_set_plane_groups(int32_t groups);

/*
 * Debug/test export: the token-plane groups G (>= 1) kq_matvec_set would
 * use for this set on the current device, or a negative KQ_ERR_* code if
 * the set is invalid (the kq_validate_set checks).  Launches nothing.
 */
int kq_debug_plan_plane_groups(const kq_tensor* tensors, int32_t n, int32_t ntok);

/* Static description of a status code (never NULL). */
const char* kq_strerror(int code);

/* ABI version of this header/library pair. */
int kq_version(void);

#define KQMV_ABI_VERSION 1

#ifdef __cplusplus
}
#endif

#endif /* KQMV_H */
