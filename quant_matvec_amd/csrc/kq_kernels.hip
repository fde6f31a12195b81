// kq_kernels.hip -- gfx950 kernels of the k-quant decode matvec.
//
// y = W x with W in k-quant super-blocks, dequantized in registers and
// never stored (muser-book Ch 13 "The QKV + gate matvec family", section
// 13.1; formats from muser-book Ch 6 sections 6.2-6.4).
//
// Mapping (one wave64 per workgroup, see kq_plan.h for the work items):
//   * lane i owns output row r0+i, so all 64 lanes walk the same super-block
//     column at the same time.  The x values a multiply-add needs are then
//     the same for the whole wave: the column's x (1 KB per token plane)
//     is written to LDS next to the weights and read back with
//     wave-uniform addresses (LDS broadcast reads).
//   * The 64 rows of a super-block column are strided in HBM (one row every
//     row_bytes).  They are fetched with coalesced 16-byte loads (one 4-byte
//     load per row and lane for the 210-byte Q6_K blocks) into registers,
//     written to a per-wave LDS slot, and read back one row per lane: a
//     transpose through LDS.  The loads of the next columns are issued before
//     the current column is computed (two columns in flight for Q4_K and
//     Q5_K, one for Q6_K).
//   * Codes become binary16 subnormals two per word (kq_decode.h) and feed
//     v_fma_mix_f32 directly, with no conversion instruction, plus about 0.6
//     (Q4_K) to 1.4 (Q6_K) bit operations per weight to unpack.
//   * Q4_K/Q5_K: every weight is formed with one rounding,
//     fma(d*sc, q, -dmin*m) (the pages' single-rounding form, muser-book
//     Ch 13 section 13.4.2), then multiplied into the sub-block's sum: two
//     instructions per weight at one token plane, 1 + ntok at ntok planes.
//     Q6_K: the code's -32 offset is taken off the packed codes exactly
//     (one binary16 add per two weights), the sub-block of 16 sums
//     (q-32)*x and is scaled once by d*sc.  Either way every rounding is
//     relative to |W_ij x_j|, so the error is bounded by a multiple of
//     sum_j |W_ij x_j| even where a block's terms cancel.
//   * No MFMA: at ntok <= 8 this is a streaming dot product, not a dense
//     contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include <mutex>
#include <type_traits>

#include "kq_decode.h"
#include "kq_plan.h"

namespace kq {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x8 __attribute__((ext_vector_type(8)));
typedef const __attribute__((address_space(1))) uint8_t* gbytes_t;   // global (not flat) byte pointer

__device__ __forceinline__ gbytes_t gbytes(const void* p) { return (gbytes_t)(p); }
// Global (not flat) float pointer: flat accesses would also count against
// the LDS counter and complete out of order with global loads, which makes
// the compiler wait for every load in flight after them.
typedef __attribute__((address_space(1))) float* gfloat_t;
__device__ __forceinline__ gfloat_t gfloat(float* p) { return (gfloat_t)(p); }

// Lane within the wave (workgroups of the pipelined kernel hold ten waves).
__device__ __forceinline__ int kq_lane() { return (int)(threadIdx.x & 63); }

constexpr float kTwo24 = 16777216.0f;        // undoes the 2^-24 of a subnormal code
constexpr float kTwo20 = 1048576.0f;         // ... of a high nibble left in place (16 * code * 2^-24)

// ---------------------------------------------------------------- wave sums
// DPP lane permutations (gfx9 encodings): quad_perm [1,0,3,2], [2,3,0,1],
// and row_half_mirror (lane i <-> 7-i inside each group of 8).
__device__ __forceinline__ float dpp_xor1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_xor2(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), lane));
}

// Workgroup id -> position in the stream.  Workgroups are dealt to the 8
// XCDs round-robin; this gives each XCD a contiguous run, so neighbouring
// workgroups (which share a tile, and the cache lines at their boundary)
// run on the same XCD and meet in its L2.
__device__ __forceinline__ int xcd_remap(int bid, int nblocks) {
    const int xcd = bid & 7, local = bid >> 3;
    const int base = nblocks >> 3, rem = nblocks & 7;
    return xcd * base + min(xcd, rem) + local;
}

// A copy of a kernel-argument struct fetched in one batch of scalar loads:
// the words are held in 8-dword groups that one empty asm statement takes as
// SGPR operands, so every load is issued before any is used (instead of each
// field being loaded next to its first use, a chain of round trips).
template <class S>
__device__ __forceinline__ S load_uniform(const S& src) {
    static_assert(sizeof(S) == 128, "four 8-dword groups");
    constexpr int G = sizeof(S) / 32;
    const u32x8* p = reinterpret_cast<const u32x8*>(&src);
    u32x8 g[G];
#pragma unroll
    for (int k = 0; k < G; ++k) g[k] = p[k];
    asm volatile("" : : "s"(g[0]), "s"(g[1]), "s"(g[2]), "s"(g[3]));
    S out;
    __builtin_memcpy(&out, g, sizeof(S));
    return out;
}

__device__ __forceinline__ uint4 lds_read4(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t lds_read1(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

constexpr int kBufFlags = 0x00020000;           // raw 32-bit buffer resource, no format conversion
constexpr int kNonTemporal = 2;                 // cache-policy operand of a load: nt

// Direct buffer -> LDS loads of the producer's steps: every lane reads SIZE
// bytes at byte offset off of the buffer r, the wave's 64 pieces land
// contiguously at lds + SIZE * lane, and a lane whose piece ends past the
// buffer's size reads nothing from memory (its piece of LDS is filled with
// zeros), so rows past the tensor's end need no clamp.  The offsets are the
// lanes' precomputed ones and the base is per step in scalar registers, so a
// step's addressing costs no vector instruction.  CP is the loads' cache
// policy: 0, or kNonTemporal for the weights of a launch of few steps a
// compute unit (the producer's choice).  They count in vmcnt until the bytes
// are in LDS.
template <int SIZE, int CP>
__device__ __forceinline__ void dma_buf(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t* lds) {
    static_assert(SIZE == 16 || SIZE == 4, "16- or 4-byte pieces");
    if constexpr (SIZE == 16)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, CP);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, CP);
}

// Direct global -> LDS loads of 16 bytes (the pipelined kernel's x): every
// lane reads 16 bytes at its own address g, and the wave's 64 pieces land
// contiguously at lds + 16 * lane (lds is the wave-uniform base).  They
// count in vmcnt until the bytes are in LDS.
__device__ __forceinline__ void dma16(gbytes_t g, uint8_t* lds) {
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)g,
                                     (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}

// ------------------------------------------------------------ x staging
// The x values of one super-block column (1 KB per token plane) travel with
// the weights: lane i loads x[4i..4i+3] of the next column into registers,
// writes them to the wave's LDS x slot next to the weights, and the lanes
// then read them back with wave-uniform addresses (an LDS broadcast read).
template <int NTOK>
struct XStage {
    float4 v[NTOK];
    __device__ __forceinline__ void load(const KqDesc& T, int b) {
        const int lane = kq_lane();
#pragma unroll
        for (int t = 0; t < NTOK; ++t)
            v[t] = __builtin_bit_cast(float4, *(const __attribute__((address_space(1))) u32x4*)(
                                                  gbytes(T.x) + 4 * (t * T.ldx + 256 * b + 4 * lane)));
    }
    __device__ __forceinline__ void commit(uint8_t* xslot) const {
        const int lane = kq_lane();
#pragma unroll
        for (int t = 0; t < NTOK; ++t) reinterpret_cast<float4*>(xslot + 1024 * t)[lane] = v[t];
    }
};

__device__ __forceinline__ float4 xread(const uint8_t* xslot, int t, int e) {
    return *reinterpret_cast<const float4*>(xslot + 1024 * t + 4 * e);
}

// End of one step of a block's multiply-adds: the step's accumulators are
// complete here and no LDS read of a later step moves above this point.
// With the x of the next step requested at the top of a step, this keeps two
// steps of x in registers instead of every read of a Q6_K quarter run
// hoisted to its start.
template <int N>
__device__ __forceinline__ void step_end(float (&a)[N], float (&b)[N]) {
#pragma unroll
    for (int t = 0; t < N; ++t) asm volatile("" : "+v"(a[t]), "+v"(b[t]));
    asm volatile("" : : : "memory");
}

// ------------------------------------------------------------ Q4_K / Q5_K
// Block of 144 (Q4_K) or 176 (Q5_K) bytes = 9 or 11 16-byte chunks.
// Q4_K: d|dmin, strip[12], qs[128].  Q5_K: d|dmin, strip[12], qh[32], qs[128].
template <int FMT>
struct K45 {
    static constexpr int BB = (FMT == KQ_Q4_K) ? 144 : 176;
    static constexpr int C = BB / 16;                          // chunks per row = uint4 staged per lane
    static constexpr int QS_OFF = (FMT == KQ_Q4_K) ? 16 : 48;  // byte offset of qs
    static constexpr int SUB = 32;
    static constexpr int WSLOT = kTileRows * BB;
};

// One group g of a block: sub-blocks 2g (low nibbles) and 2g+1 (high).
// Every weight is formed first, with one rounding, as the pages' fallback
// form fma(d*sc, q, -dmin*m) (muser-book Ch 13 section 13.4.2; Ch 6 section
// 6.2): d*sc and dmin*m are exact in float32 (11 x 6 significant bits), and
// so is (d*sc)*q, so the weight is the exact value correctly rounded, and a
// weight that is exactly zero stays zero.  The code enters v_fma_mix_f32 as
// its binary16 subnormal (code * 2^-24, or code * 2^-20 for a high nibble
// left in place); the 2^24 / 2^20 is folded into d*sc.  Then sum_e W_e x_e
// per sub-block: every rounding is relative to |W_e x_e|, so the result's
// error is bounded by a multiple of sum_j |W_ij x_j| (no separate min term
// that could cancel against the code term).
template <int FMT, int NTOK, int G>
__device__ __forceinline__ void k45_group(const uint32_t (&qs)[8], const uint32_t (&qh)[8], const K4Scales& S, float d,
                                          float dmin, const uint8_t* xslot, float (&c)[NTOK]) {
    const float a_lo = d * (float)k4_sc(S, 2 * G) * kTwo24;          // exact
    const float a_hi = d * (float)k4_sc(S, 2 * G + 1) * kTwo20;
    const float n_lo = -(dmin * (float)k4_m(S, 2 * G));               // exact
    const float n_hi = -(dmin * (float)k4_m(S, 2 * G + 1));
    float al[NTOK], ah[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) { al[t] = 0.0f; ah[t] = 0.0f; }
    // The weights of step k (elements 64G + 4k + i and 64G + 32 + 4k + i),
    // multiplied into al / ah with that step's x.
    auto step = [&](int k, const float4 (&xl)[NTOK], const float4 (&xh)[NTOK]) {
        Packed4 p;
        if constexpr (FMT == KQ_Q4_K) p = k4_codes(qs[k]);
        else p = k5_codes<G>(qs[k], qh[k]);
        const float wl0 = __builtin_fmaf(a_lo, (float)half_lo(p.lo02), n_lo);
        const float wl1 = __builtin_fmaf(a_lo, (float)half_lo(p.lo13), n_lo);
        const float wl2 = __builtin_fmaf(a_lo, (float)half_hi(p.lo02), n_lo);
        const float wl3 = __builtin_fmaf(a_lo, (float)half_hi(p.lo13), n_lo);
        const float wh0 = __builtin_fmaf(a_hi, (float)half_lo(p.hi02), n_hi);
        const float wh1 = __builtin_fmaf(a_hi, (float)half_lo(p.hi13), n_hi);
        const float wh2 = __builtin_fmaf(a_hi, (float)half_hi(p.hi02), n_hi);
        const float wh3 = __builtin_fmaf(a_hi, (float)half_hi(p.hi13), n_hi);
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            al[t] = __builtin_fmaf(wl0, xl[t].x, al[t]);
            al[t] = __builtin_fmaf(wl1, xl[t].y, al[t]);
            al[t] = __builtin_fmaf(wl2, xl[t].z, al[t]);
            al[t] = __builtin_fmaf(wl3, xl[t].w, al[t]);
            ah[t] = __builtin_fmaf(wh0, xh[t].x, ah[t]);
            ah[t] = __builtin_fmaf(wh1, xh[t].y, ah[t]);
            ah[t] = __builtin_fmaf(wh2, xh[t].z, ah[t]);
            ah[t] = __builtin_fmaf(wh3, xh[t].w, ah[t]);
        }
    };
    if constexpr (NTOK <= 2) {
        // x of step k in buffer k % 2, read one step ahead; step_end keeps
        // later reads from being hoisted (the registers of a whole group's
        // x would not fit beside the rest)
        float4 xb[2][2][NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            xb[0][0][t] = xread(xslot, t, 64 * G);
            xb[0][1][t] = xread(xslot, t, 64 * G + 32);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (k + 1 < 8) {
#pragma unroll
                for (int t = 0; t < NTOK; ++t) {
                    xb[(k + 1) % 2][0][t] = xread(xslot, t, 64 * G + 4 * (k + 1));
                    xb[(k + 1) % 2][1][t] = xread(xslot, t, 64 * G + 32 + 4 * (k + 1));
                }
            }
            step(k, xb[k % 2][0], xb[k % 2][1]);
            step_end<NTOK>(al, ah);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            Packed4 p;
            if constexpr (FMT == KQ_Q4_K) p = k4_codes(qs[k]);
            else p = k5_codes<G>(qs[k], qh[k]);
            const int e = 64 * G + 4 * k;
            const float wl0 = __builtin_fmaf(a_lo, (float)half_lo(p.lo02), n_lo);
            const float wl1 = __builtin_fmaf(a_lo, (float)half_lo(p.lo13), n_lo);
            const float wl2 = __builtin_fmaf(a_lo, (float)half_hi(p.lo02), n_lo);
            const float wl3 = __builtin_fmaf(a_lo, (float)half_hi(p.lo13), n_lo);
            const float wh0 = __builtin_fmaf(a_hi, (float)half_lo(p.hi02), n_hi);
            const float wh1 = __builtin_fmaf(a_hi, (float)half_lo(p.hi13), n_hi);
            const float wh2 = __builtin_fmaf(a_hi, (float)half_hi(p.hi02), n_hi);
            const float wh3 = __builtin_fmaf(a_hi, (float)half_hi(p.hi13), n_hi);
#pragma unroll
            for (int t = 0; t < NTOK; ++t) {
                const float4 xl = xread(xslot, t, e), xh = xread(xslot, t, e + 32);
                al[t] = __builtin_fmaf(wl0, xl.x, al[t]);
                al[t] = __builtin_fmaf(wl1, xl.y, al[t]);
                al[t] = __builtin_fmaf(wl2, xl.z, al[t]);
                al[t] = __builtin_fmaf(wl3, xl.w, al[t]);
                ah[t] = __builtin_fmaf(wh0, xh.x, ah[t]);
                ah[t] = __builtin_fmaf(wh1, xh.y, ah[t]);
                ah[t] = __builtin_fmaf(wh2, xh.z, ah[t]);
                ah[t] = __builtin_fmaf(wh3, xh.w, ah[t]);
            }
        }
    }
#pragma unroll
    for (int t = 0; t < NTOK; ++t) c[t] = (c[t] + al[t]) + ah[t];
}

// The qs words of group G of a block at `row` (LDS).
template <int FMT, int G>
__device__ __forceinline__ void k45_qs(const uint8_t* row, uint32_t (&qs)[8]) {
    const uint4 a = lds_read4(row + K45<FMT>::QS_OFF + 32 * G);
    const uint4 b = lds_read4(row + K45<FMT>::QS_OFF + 32 * G + 16);
    qs[0] = a.x; qs[1] = a.y; qs[2] = a.z; qs[3] = a.w;
    qs[4] = b.x; qs[5] = b.y; qs[6] = b.z; qs[7] = b.w;
}

// The block's contribution from its header, qh words and the qs words of
// each group (read by the caller into qs[G]), formed from zero (sub-blocks
// 0..7 summed in order) and then added to acc, so that a block adds the
// same bits in either tile height and from LDS or registers.
template <int FMT, int NTOK, class QS>
__device__ __forceinline__ void k45_block(const uint4& hdr, const uint32_t (&qh)[8], const QS& qs_of,
                                          const uint8_t* xslot, float (&acc)[NTOK]) {
    const float d = f16_to_f32(hdr.x & 0xFFFFu), dmin = f16_to_f32(hdr.x >> 16);
    const K4Scales S = k4_scales(hdr.y, hdr.z, hdr.w);
    float c[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) c[t] = 0.0f;
    uint32_t qs[8];
    qs_of(qs, std::integral_constant<int, 0>());
    k45_group<FMT, NTOK, 0>(qs, qh, S, d, dmin, xslot, c);
    qs_of(qs, std::integral_constant<int, 1>());
    k45_group<FMT, NTOK, 1>(qs, qh, S, d, dmin, xslot, c);
    qs_of(qs, std::integral_constant<int, 2>());
    k45_group<FMT, NTOK, 2>(qs, qh, S, d, dmin, xslot, c);
    qs_of(qs, std::integral_constant<int, 3>());
    k45_group<FMT, NTOK, 3>(qs, qh, S, d, dmin, xslot, c);
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = acc[t] + c[t];
}

// acc[t] += the contribution of the Q4_K/Q5_K block at `row` (LDS) with x
// at xslot.
template <int FMT, int NTOK>
__device__ __forceinline__ void block_mac(const uint8_t* row, const uint8_t* xslot, float (&acc)[NTOK]) {
    const uint4 hdr = lds_read4(row);
    uint32_t qh[8];
    if constexpr (FMT == KQ_Q5_K) {
        const uint4 a = lds_read4(row + 16), c = lds_read4(row + 32);
        qh[0] = a.x; qh[1] = a.y; qh[2] = a.z; qh[3] = a.w;
        qh[4] = c.x; qh[5] = c.y; qh[6] = c.z; qh[7] = c.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = 0;
    }
    k45_block<FMT, NTOK>(hdr, qh, [&](uint32_t (&qs)[8], auto g) { k45_qs<FMT, decltype(g)::value>(row, qs); },
                         xslot, acc);
}

// The same from the block's bytes held in registers (wv: the block's 16-byte
// chunks, as it lies in memory).
template <int FMT, int NTOK>
__device__ __forceinline__ void block_mac_regs(const uint4 (&wv)[K45<FMT>::C], const uint8_t* xslot,
                                               float (&acc)[NTOK]) {
    uint32_t qh[8];
    if constexpr (FMT == KQ_Q5_K) {
        qh[0] = wv[1].x; qh[1] = wv[1].y; qh[2] = wv[1].z; qh[3] = wv[1].w;
        qh[4] = wv[2].x; qh[5] = wv[2].y; qh[6] = wv[2].z; qh[7] = wv[2].w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) qh[i] = 0;
    }
    constexpr int Q = K45<FMT>::QS_OFF / 16;
    k45_block<FMT, NTOK>(wv[0], qh, [&](uint32_t (&qs)[8], auto g) {
        constexpr int G = decltype(g)::value;
        const uint4 a = wv[Q + 2 * G], b = wv[Q + 2 * G + 1];
        qs[0] = a.x; qs[1] = a.y; qs[2] = a.z; qs[3] = a.w;
        qs[4] = b.x; qs[5] = b.y; qs[6] = b.z; qs[7] = b.w;
    }, xslot, acc);
}

// Per-lane staging offsets of a 64-row column: 16-byte chunk q = 64*i + lane
// of the column is row q / C, chunk q % C, at byte offset row*row_bytes +
// 16*chunk from the tile's first row; in LDS it lands at byte 16*q =
// row*BB + 16*chunk.
template <int C>
struct K45Offsets {
    uint32_t off[C];
    __device__ __forceinline__ void init(const KqDesc& T) {
        int lane = kq_lane();
        // opaque to the optimizer, so these per-format offsets are formed
        // here and not hoisted to the kernel entry for every format
        asm volatile("" : "+v"(lane));
#pragma unroll
        for (int i = 0; i < C; ++i) {
            const int q = 64 * i + lane;
            const int r = q / C, c = q - (q / C) * C;
            off[i] = (uint32_t)r * (uint32_t)T.row_bytes + 16u * c;
        }
    }
};

// Staging and compute of one super-block column of 64 rows.
template <int FMT, int NTOK>
struct K45Column {
    static constexpr int TR = kTileRows, CPS = 1;               // tile rows, columns a step
    static constexpr int C = K45<FMT>::C;
    static constexpr int BB = K45<FMT>::BB;
    typedef K45Offsets<C> Offsets;
    uint4 stg[C];
    XStage<NTOK> xs;

    // Loads are branch-free: chunks of rows past the end of the tensor (in
    // its last tile) are clamped to the last chunk of its last row, which
    // every such chunk exceeds, so they read valid memory whose values are
    // never used.
    // `valid` false: the column lies past the run; every lane then reads the
    // tensor's first 16 bytes (values unused), so that the loads and the
    // registers they fill are the same on every path.
    __device__ __forceinline__ void stage(const KqDesc& T, const Offsets& o, int tile, int b, bool valid) {
        const int rows_here = min(kTileRows, T.rows - tile * kTileRows);
        const uint32_t max_off = valid ? (uint32_t)(rows_here - 1) * (uint32_t)T.row_bytes + 16u * (C - 1) : 0u;
        gbytes_t col = gbytes(T.w) + (valid ? (size_t)tile * kTileRows * T.row_bytes + (size_t)b * BB : (size_t)0);
#pragma unroll
        for (int i = 0; i < C; ++i)
            stg[i] = __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(col + min(o.off[i], max_off)));
        xs.load(T, valid ? b : 0);
    }
    __device__ __forceinline__ void commit(uint8_t* slot) const {
        const int lane = kq_lane();
#pragma unroll
        for (int i = 0; i < C; ++i) reinterpret_cast<uint4*>(slot)[64 * i + lane] = stg[i];
        xs.commit(slot + K45<FMT>::WSLOT);
    }
    // acc[t] += this column's contribution for the lane's row (formed on
    // its own first, as a 32-row tile forms each block's, so that a segment
    // sums to the same bits in either tile height)
    static __device__ __forceinline__ void compute(const KqDesc& T, const uint8_t* slot, int tile, int b,
                                                   float (&acc)[NTOK]) {
        (void)T; (void)tile; (void)b;
        block_mac<FMT, NTOK>(slot + kq_lane() * BB, slot + K45<FMT>::WSLOT, acc);
    }
};

// A 32-row tile of a Q4_K/Q5_K matrix, one segment (blocks b, b+1) a step.
// Chunk q = 64*i + lane of a step is row q / 2C, 16-byte chunk q % 2C of the
// row's two blocks (contiguous in memory), and lands in LDS at byte 16*q,
// so row r's two blocks sit at r*2*BB and r*2*BB + BB.  Lane 2r + k
// computes block b + k of row r, with column b + k's x.
template <int FMT, int NTOK>
struct K45Pair {
    static constexpr int TR = 32, CPS = 2;                     // tile rows, columns a step
    static constexpr int C = K45<FMT>::C, BB = K45<FMT>::BB, C2 = 2 * C;
    static constexpr int N = TR * C2 / 64;                     // loads a lane: C
    static constexpr int WSLOT = TR * 2 * BB;
    struct Offsets {
        uint32_t off[N];
        __device__ __forceinline__ void init(const KqDesc& T) {
            int lane = kq_lane();
            asm volatile("" : "+v"(lane));
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const int q = 64 * i + lane;
                const int r = q / C2, c = q - (q / C2) * C2;
                off[i] = (uint32_t)r * (uint32_t)T.row_bytes + 16u * c;
            }
        }
    };
    uint4 stg[N];
    XStage<NTOK> xs0, xs1;
    // ---- the pipelined kernel's pieces: the step's weights go to an LDS
    // slot by direct loads, in commit()'s layout (chunk q at byte 16q); x
    // (block b, then b+1, one plane per token) sits in a slot of its own; a
    // consumer reads its lane's block into registers, frees the weight
    // slot, and computes from registers
    static constexpr int LOADS = N;                            // direct loads of one step
    static constexpr int PC_W = WSLOT, PC_X = 2 * 1024 * NTOK; // LDS bytes of a step's weights, x
    // The step's buffer starts at block b of the tile's first row and ends
    // with block b + 1 of its last row in the tensor.
    template <int CP>
    static __device__ __forceinline__ void dma_w(const KqDesc& T, const Offsets& o, int tile, int b, uint8_t* wslot) {
        const int rows_here = min(TR, T.rows - tile * TR);
        const int64_t base = (int64_t)tile * TR * T.row_bytes + (int64_t)b * BB;
        const int size = rows_here * (int)T.row_bytes - b * BB;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)(T.w + base), (short)0, size, kBufFlags);
#pragma unroll
        for (int i = 0; i < N; ++i) kq::dma_buf<16, CP>(r, o.off[i], wslot + 1024 * i);
    }
    struct Regs {
        uint4 v[C];
    };
    static __device__ __forceinline__ void load_regs(const uint8_t* wslot, Regs& r) {
        const int lane = kq_lane();
        const uint8_t* blk = wslot + (lane >> 1) * 2 * BB + (lane & 1) * BB;
#pragma unroll
        for (int i = 0; i < C; ++i) r.v[i] = lds_read4(blk + 16 * i);
    }
    static __device__ __forceinline__ void compute_regs(const Regs& r, const uint8_t* xslot, float (&acc)[NTOK]) {
        block_mac_regs<FMT, NTOK>(r.v, xslot + (kq_lane() & 1) * 1024 * NTOK, acc);
    }

    // Branch-free, clamped like the 64-row column (rows past the tensor's
    // end read its last row's last chunk; `valid` false reads the tensor's
    // first bytes and x of columns 0 and 1, which every such tensor has).
    __device__ __forceinline__ void stage(const KqDesc& T, const Offsets& o, int tile, int b, bool valid) {
        const int rows_here = min(TR, T.rows - tile * TR);
        const uint32_t max_off = valid ? (uint32_t)(rows_here - 1) * (uint32_t)T.row_bytes + 16u * (C2 - 1) : 0u;
        gbytes_t col = gbytes(T.w) + (valid ? (size_t)tile * TR * T.row_bytes + (size_t)b * BB : (size_t)0);
#pragma unroll
        for (int i = 0; i < N; ++i)
            stg[i] = __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(col + min(o.off[i], max_off)));
        xs0.load(T, valid ? b : 0);
        xs1.load(T, valid ? b + 1 : 1);
    }
    __device__ __forceinline__ void commit(uint8_t* slot) const {
        const int lane = kq_lane();
#pragma unroll
        for (int i = 0; i < N; ++i) reinterpret_cast<uint4*>(slot)[64 * i + lane] = stg[i];
        xs0.commit(slot + WSLOT);
        xs1.commit(slot + WSLOT + 1024 * NTOK);
    }
    static __device__ __forceinline__ void compute(const KqDesc& T, const uint8_t* slot, int tile, int b,
                                                   float (&acc)[NTOK]) {
        (void)T; (void)tile; (void)b;
        const int lane = kq_lane(), k = lane & 1;
        block_mac<FMT, NTOK>(slot + (lane >> 1) * 2 * BB + k * BB, slot + WSLOT + k * 1024 * NTOK, acc);
    }
};

// -------------------------------------------------------------------- Q6_K
// 210-byte block: ql[128], qh[64], sc[16] (int8), d (f16, last).  A block
// starts 2 bytes into a word when its index in the tensor is odd, so each
// row's block is staged as the 53 aligned words covering it: words 0..51 as
// 13 16-byte chunks (a column is 13 load instructions of 64 chunks, like
// the Q4_K/Q5_K path) into a 208-byte LDS row, and word 52 (lane = row) into
// a separate 64-word array.  The compute shifts by two bytes where needed.
constexpr int kQ6Chunks = 13;
constexpr int kQ6LdsRow = 16 * kQ6Chunks;     // 208: 52 words, odd multiple of 4 -> conflict-free rows

// The block's words w[i..i+3] (and w[i+4] for the shift) realigned.
__device__ __forceinline__ void q6_read4(const uint8_t* row, int i, uint32_t sh, uint32_t (&o)[4]) {
    const uint4 a = lds_read4(row + 4 * i);
    const uint32_t e = lds_read1(row + 4 * i + 16);
    o[0] = __builtin_amdgcn_alignbit(a.y, a.x, sh);
    o[1] = __builtin_amdgcn_alignbit(a.z, a.y, sh);
    o[2] = __builtin_amdgcn_alignbit(a.w, a.z, sh);
    o[3] = __builtin_amdgcn_alignbit(e, a.w, sh);
}

// The signed Q6_K code q - 32 of both halves of a packed pair: the halves
// are binary16 subnormals (code or 16*code times 2^-24) and the offset is
// subtracted as binary16 (neg = -32 or -512 times 2^-24 in both halves).
// The difference is a multiple of 2^-24 below 2^-14 in magnitude, so the
// subtraction is exact and yields the signed subnormal (q-32) * 2^-24 (or
// 16*(q-32) * 2^-24).
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t q6_signed(uint32_t p, uint32_t neg) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, p) + __builtin_bit_cast(half2_t, neg));
}
constexpr uint32_t kQ6NegLo = 0x80208020u;    // -32 * 2^-24 in both halves
constexpr uint32_t kQ6NegHi = 0x82008200u;    // -512 * 2^-24: the offset of a high nibble left in place

// Sixteen elements l = 16KH..16KH+15 of each quarter c of half N (elements
// 128N + 32c + l, sub-block 8N + 2c + KH of 16): for each quarter the sum
// of (q-32)*x over the sub-block, scaled by its int8 scale, goes to tl
// (quarters 0, 1: codes at 2^-24) or th (quarters 2, 3: at 2^-20).  The
// code carries its offset (q6_signed), so every rounding is relative to
// |W_e x_e| and nothing is subtracted after the sum.
template <int NTOK, int N, int KH>
__device__ __forceinline__ void q6_quarter_run(const uint32_t (&A)[4], const uint32_t (&B)[4], const uint32_t (&H)[4],
                                               const uint32_t (&scw)[4], const uint8_t* xslot, float (&tl)[NTOK],
                                               float (&th)[NTOK]) {
    // A: ql bytes 64N + 16KH.., B: ql bytes 64N + 32 + 16KH.., H: qh bytes
    // 32N + 16KH.. (realigned words)
    float a[4][NTOK];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < NTOK; ++t) a[c][t] = 0.0f;
    if constexpr (NTOK <= 2) {
        // x of step kk (elements 128N + 32c + 4k, c = 0..3) sits in buffer
        // kk % 2, requested one step ahead
        float4 xb[2][4][NTOK];
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int t = 0; t < NTOK; ++t) xb[0][c][t] = xread(xslot, t, 128 * N + 32 * c + 4 * (4 * KH));
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int k = 4 * KH + kk;
            if (kk + 1 < 4) {
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int t = 0; t < NTOK; ++t) xb[(kk + 1) % 2][c][t] = xread(xslot, t, 128 * N + 32 * c + 4 * (k + 1));
            }
            Packed6 p = k6_codes(A[kk], B[kk], H[kk]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                p.c02[c] = q6_signed(p.c02[c], c < 2 ? kQ6NegLo : kQ6NegHi);
                p.c13[c] = q6_signed(p.c13[c], c < 2 ? kQ6NegLo : kQ6NegHi);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
#pragma unroll
                for (int t = 0; t < NTOK; ++t) {
                    const float4 xv = xb[kk % 2][c][t];
                    a[c][t] = __builtin_fmaf((float)half_lo(p.c02[c]), xv.x, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_lo(p.c13[c]), xv.y, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_hi(p.c02[c]), xv.z, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_hi(p.c13[c]), xv.w, a[c][t]);
                }
            }
            step_end<NTOK>(a[0], a[1]);
            step_end<NTOK>(a[2], a[3]);
        }
    } else {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int k = 4 * KH + kk;
            Packed6 p = k6_codes(A[kk], B[kk], H[kk]);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                p.c02[c] = q6_signed(p.c02[c], c < 2 ? kQ6NegLo : kQ6NegHi);
                p.c13[c] = q6_signed(p.c13[c], c < 2 ? kQ6NegLo : kQ6NegHi);
            }
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const int e = 128 * N + 32 * c + 4 * k;
#pragma unroll
                for (int t = 0; t < NTOK; ++t) {
                    const float4 xv = xread(xslot, t, e);
                    a[c][t] = __builtin_fmaf((float)half_lo(p.c02[c]), xv.x, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_lo(p.c13[c]), xv.y, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_hi(p.c02[c]), xv.z, a[c][t]);
                    a[c][t] = __builtin_fmaf((float)half_hi(p.c13[c]), xv.w, a[c][t]);
                }
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = 8 * N + 2 * c + KH;                                   // sub-block of 16
        const float scj = (float)(int8_t)(scw[j / 4] >> (8 * (j % 4)));
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            if (c < 2) tl[t] = __builtin_fmaf(scj, a[c][t], tl[t]);
            else th[t] = __builtin_fmaf(scj, a[c][t], th[t]);
        }
    }
}

// The Q6_K block's contribution from its scale words 48..51, word 52 (scales
// 14-15 and d, or d alone) and, per quarter run (N, KH), the realigned ql
// and qh words that words(N, KH, A, B, H) fetches; formed from zero and
// then added to acc, so that a block adds the same bits in either tile
// height and from LDS or registers.
template <int NTOK, class W>
__device__ __forceinline__ void q6_block(uint32_t s48, uint32_t s49, uint32_t s50, uint32_t s51, uint32_t w52,
                                         uint32_t sh, const W& words, const uint8_t* xslot, float (&acc)[NTOK]) {
    uint32_t scw[4];
    scw[0] = __builtin_amdgcn_alignbit(s49, s48, sh);
    scw[1] = __builtin_amdgcn_alignbit(s50, s49, sh);
    scw[2] = __builtin_amdgcn_alignbit(s51, s50, sh);
    scw[3] = __builtin_amdgcn_alignbit(w52, s51, sh);
    const float d = f16_to_f32((w52 >> sh) & 0xFFFFu);
    float tl[NTOK], th[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) { tl[t] = 0.0f; th[t] = 0.0f; }
    uint32_t A[4], B[4], H[4];
    using Z = std::integral_constant<int, 0>;
    using O = std::integral_constant<int, 1>;
    words(Z(), Z(), A, B, H);
    q6_quarter_run<NTOK, 0, 0>(A, B, H, scw, xslot, tl, th);
    words(Z(), O(), A, B, H);
    q6_quarter_run<NTOK, 0, 1>(A, B, H, scw, xslot, tl, th);
    words(O(), Z(), A, B, H);
    q6_quarter_run<NTOK, 1, 0>(A, B, H, scw, xslot, tl, th);
    words(O(), O(), A, B, H);
    q6_quarter_run<NTOK, 1, 1>(A, B, H, scw, xslot, tl, th);
    const float d24 = d * kTwo24;
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = acc[t] + d24 * __builtin_fmaf(th[t], 0.0625f, tl[t]);
}

// acc[t] += the contribution of the Q6_K block whose aligned words start at
// `row` (LDS), shifted by sh bits, with word 52 given apart; x at xslot.
// The block's sum is formed from zero and then added, so that a block adds
// the same bits in either tile height.
template <int NTOK>
__device__ __forceinline__ void q6_block_mac(const uint8_t* row, uint32_t w52, uint32_t sh, const uint8_t* xslot,
                                             float (&acc)[NTOK]) {
    // words 48..51 (scales) and word 52 (scales 14-15 and d, or d alone)
    const uint4 s4 = lds_read4(row + 4 * 48);
    q6_block<NTOK>(s4.x, s4.y, s4.z, s4.w, w52, sh, [&](auto n, auto kh, uint32_t (&A)[4], uint32_t (&B)[4],
                                                        uint32_t (&H)[4]) {
        constexpr int N = decltype(n)::value, KH = decltype(kh)::value;
        q6_read4(row, 16 * N + 4 * KH, sh, A);
        q6_read4(row, 16 * N + 8 + 4 * KH, sh, B);
        q6_read4(row, 32 + 8 * N + 4 * KH, sh, H);
    }, xslot, acc);
}

// The same from the block's 53 aligned words held in registers (wd[i] =
// word i of the block's aligned span, shifted by sh bits).
template <int NTOK>
__device__ __forceinline__ void q6_block_mac_regs(const uint32_t (&wd)[53], uint32_t sh, const uint8_t* xslot,
                                                  float (&acc)[NTOK]) {
    q6_block<NTOK>(wd[48], wd[49], wd[50], wd[51], wd[52], sh, [&](auto n, auto kh, uint32_t (&A)[4],
                                                                   uint32_t (&B)[4], uint32_t (&H)[4]) {
        constexpr int N = decltype(n)::value, KH = decltype(kh)::value;
        constexpr int ia = 16 * N + 4 * KH, ib = 16 * N + 8 + 4 * KH, ih = 32 + 8 * N + 4 * KH;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            A[q] = __builtin_amdgcn_alignbit(wd[ia + q + 1], wd[ia + q], sh);
            B[q] = __builtin_amdgcn_alignbit(wd[ib + q + 1], wd[ib + q], sh);
            H[q] = __builtin_amdgcn_alignbit(wd[ih + q + 1], wd[ih + q], sh);
        }
    }, xslot, acc);
}

// Per-lane staging offsets of a 64-row Q6_K column.  Chunk q = 64*i + lane
// is row q / 13, words 4*(q % 13).. of that row's aligned span; word 52 of
// row `lane` is one more dword load.  With an even number of blocks per row
// (row_bytes a multiple of 4) every row of a column has the same alignment.
// With an odd number (ALT) it alternates between rows: an odd row's aligned
// start sits 2 bytes away from row_bytes * row, in the direction that row
// 0's alignment gives (`corr`, set per column); bit i of `odd` marks chunk
// i's row as odd, bit 13 the lane's own row.
template <bool ALT>
struct Q6Offsets {
    uint32_t off[kQ6Chunks];
    uint32_t off52;
    uint32_t odd;
    __device__ __forceinline__ void init(const KqDesc& T) {
        int lane = kq_lane();
        asm volatile("" : "+v"(lane));
        const uint32_t rb = (uint32_t)T.row_bytes;
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < kQ6Chunks; ++i) {
            const uint32_t q = 64u * i + (uint32_t)lane;
            const uint32_t r = q / kQ6Chunks, c = q - r * kQ6Chunks;
            off[i] = r * rb + 16u * c;
            m |= (r & 1u) << i;
        }
        off52 = (uint32_t)lane * rb + 208u;
        odd = ALT ? (m | (((uint32_t)lane & 1u) << 13)) : 0u;
    }
    // offset of chunk i (13: word 52) for a column whose odd rows move by corr
    __device__ __forceinline__ uint32_t at(int i, int32_t corr) const {
        const uint32_t o = i < kQ6Chunks ? off[i] : off52;
        if constexpr (!ALT) return o;
        return o + (uint32_t)((int32_t)((odd >> i) & 1u) * corr);
    }
};

template <int NTOK, bool ALT>
struct Q6Column {
    static constexpr int TR = kTileRows, CPS = 1;               // tile rows, columns a step
    static constexpr int WSLOT = kTileRows * kQ6LdsRow + 4 * kTileRows;
    typedef Q6Offsets<ALT> Offsets;
    uint4 stg[kQ6Chunks];
    uint32_t w52;         // word 52 of the lane's row
    uint32_t tailv;       // bytes 208-209 of the tensor's last block (tail case)
    int tail_row;         // its row in the tile, or -1
    XStage<NTOK> xs;

    // Branch-free.  Chunks of rows past the tensor's end are clamped to the
    // last chunk of its last row (every such chunk's offset exceeds it).
    // The tensor's very last block, when it starts 4-byte aligned, ends 2
    // bytes into its word 52: that row reads its word 51 instead, and bytes
    // 208-209 are read on their own and put in its place at the commit.
    // `valid` false: the column lies past the run; every lane then reads the
    // tensor's first bytes (values unused).
    __device__ __forceinline__ void stage(const KqDesc& T, const Offsets& o, int tile, int b, bool valid) {
        const int r0 = tile * kTileRows;
        const int last_row = min(kTileRows, T.rows - r0) - 1;
        const int32_t rb = (int32_t)T.row_bytes;
        const int64_t start = (int64_t)r0 * T.row_bytes + 210 * (int64_t)b;    // row r0's block
        const int64_t last = start + (int64_t)last_row * T.row_bytes;         // the tile's last row's block
        const bool tail = valid && (r0 + last_row + 1 == T.rows) && (b == T.nb - 1) && ((last & 3) == 0);
        const int32_t corr = ALT ? 2 * (int32_t)(start & 3) - 2 : 0;
        const int32_t dl = (last_row & 1) ? corr : 0;
        uint32_t max_off = valid ? (uint32_t)(last_row * rb + 16 * (kQ6Chunks - 1) + dl) : 0u;
        uint32_t max52 = valid ? (uint32_t)(last_row * rb + (tail ? 204 : 208) + dl) : 0u;
        asm volatile("" : "+s"(max_off), "+s"(max52));
        gbytes_t col = gbytes(T.w) + (valid ? (start & ~(int64_t)3) : 0);
#pragma unroll
        for (int i = 0; i < kQ6Chunks; ++i)
            stg[i] = __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(
                                                  col + min(o.at(i, corr), max_off)));
        w52 = *(const __attribute__((address_space(1))) uint32_t*)(col + min(o.at(kQ6Chunks, corr), max52));
        tail_row = tail ? last_row : -1;
        tailv = *(const __attribute__((address_space(1))) uint16_t*)(gbytes(T.w) + (tail ? last + 208 : 0));
        xs.load(T, valid ? b : 0);
    }
    __device__ __forceinline__ void commit(uint8_t* slot) const {
        const int lane = kq_lane();
#pragma unroll
        for (int i = 0; i < kQ6Chunks; ++i) reinterpret_cast<uint4*>(slot)[64 * i + lane] = stg[i];
        reinterpret_cast<uint32_t*>(slot + kTileRows * kQ6LdsRow)[lane] = lane == tail_row ? tailv : w52;
        xs.commit(slot + WSLOT);
    }
    static __device__ __forceinline__ void compute(const KqDesc& T, const uint8_t* slot, int tile, int b,
                                                   float (&acc)[NTOK]) {
        const int lane = kq_lane();
        // the block starts 2 bytes into its first staged word when its index
        // in the tensor, (r0+lane)*nb + b, is odd
        const uint32_t sh = !ALT ? 16u * (uint32_t)(b & 1)
                                 : 16u * (uint32_t)(((int64_t)(tile * kTileRows + lane) * T.nb + b) & 1);
        q6_block_mac<NTOK>(slot + lane * kQ6LdsRow, lds_read1(slot + kTileRows * kQ6LdsRow + 4 * lane), sh,
                           slot + WSLOT, acc);
    }
};

// A 32-row tile of a Q6_K matrix with an even number of blocks a row, one
// segment (blocks b, b+1, b even) a step.  A row's two blocks are 420 bytes
// from a 4-byte-aligned start: words 0..103 go as 26 16-byte chunks
// (chunk q = 64*i + lane of the step is row q / 26, chunk q % 26; it lands
// at LDS byte 16*q), word 104 (lane = row) into a separate 32-word array.
// Lane 2r + k computes block b + k of row r: block b from word 0, block b+1
// from word 52 two bytes in; its word 52 is the pair's word 104.  The pair
// ends where the row does, so nothing past the tensor is read.
template <int NTOK>
struct Q6Pair {
    static constexpr int TR = 32, CPS = 2;                     // tile rows, columns a step
    static constexpr int CH = 26;                              // chunks of a row's pair
    static constexpr int ROWB = 16 * CH;                       // 416: odd multiple of 16
    static constexpr int N = TR * CH / 64;                     // loads a lane: 13
    static constexpr int WSLOT = TR * ROWB + 4 * 64;           // word 104 of each lane's row, then x
    struct Offsets {
        uint32_t off[N];
        uint32_t off104;
        __device__ __forceinline__ void init(const KqDesc& T) {
            int lane = kq_lane();
            asm volatile("" : "+v"(lane));
            const uint32_t rb = (uint32_t)T.row_bytes;
#pragma unroll
            for (int i = 0; i < N; ++i) {
                const uint32_t q = 64u * i + (uint32_t)lane;
                const uint32_t r = q / CH, c = q - r * CH;
                off[i] = r * rb + 16u * c;
            }
            off104 = ((uint32_t)lane & 31u) * rb + 416u;
        }
    };
    uint4 stg[N];
    uint32_t w104;
    XStage<NTOK> xs0, xs1;
    // ---- the pipelined kernel's pieces (as in K45Pair): word 104 of row
    // (lane & 31) lands at word `lane` of its array (lanes 32..63 repeat
    // rows 0..31); a lane's block is 53 aligned words, shifted 16 bits for
    // the pair's second block
    static constexpr int LOADS = N + 1;                        // direct loads of one step
    static constexpr int PC_W = WSLOT, PC_X = 2 * 1024 * NTOK; // LDS bytes of a step's weights, x
    // The step's buffer starts at the pair's first byte in the tile's first
    // row (4-byte aligned: b is even) and ends with the pair of its last row
    // in the tensor.
    template <int CP>
    static __device__ __forceinline__ void dma_w(const KqDesc& T, const Offsets& o, int tile, int b, uint8_t* wslot) {
        const int rows_here = min(TR, T.rows - tile * TR);
        const int64_t base = (int64_t)tile * TR * T.row_bytes + (int64_t)210 * b;
        const int size = rows_here * (int)T.row_bytes - 210 * b;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)(T.w + base), (short)0, size, kBufFlags);
#pragma unroll
        for (int i = 0; i < N; ++i) kq::dma_buf<16, CP>(r, o.off[i], wslot + 1024 * i);
        kq::dma_buf<4, CP>(r, o.off104, wslot + TR * ROWB);
    }
    struct Regs {
        uint32_t wd[53];
    };
    static __device__ __forceinline__ void load_regs(const uint8_t* wslot, Regs& r) {
        const int lane = kq_lane(), k = lane & 1, rr = lane >> 1;
        const uint8_t* rowp = wslot + rr * ROWB + k * 208;
#pragma unroll
        for (int i = 0; i < 13; ++i) {
            const uint4 q = lds_read4(rowp + 16 * i);
            r.wd[4 * i] = q.x; r.wd[4 * i + 1] = q.y; r.wd[4 * i + 2] = q.z; r.wd[4 * i + 3] = q.w;
        }
        r.wd[52] = lds_read1(k ? wslot + TR * ROWB + 4 * rr : rowp + 208);
    }
    static __device__ __forceinline__ void compute_regs(const Regs& r, const uint8_t* xslot, float (&acc)[NTOK]) {
        const int k = kq_lane() & 1;
        q6_block_mac_regs<NTOK>(r.wd, k ? 16u : 0u, xslot + k * 1024 * NTOK, acc);
    }

    __device__ __forceinline__ void stage(const KqDesc& T, const Offsets& o, int tile, int b, bool valid) {
        const int rows_here = min(TR, T.rows - tile * TR);
        const uint32_t rb = (uint32_t)T.row_bytes;
        const uint32_t max_off = valid ? (uint32_t)(rows_here - 1) * rb + 16u * (CH - 1) : 0u;
        const uint32_t max104 = valid ? (uint32_t)(rows_here - 1) * rb + 416u : 0u;
        gbytes_t col = gbytes(T.w) + (valid ? (size_t)tile * TR * T.row_bytes + (size_t)210 * b : (size_t)0);
#pragma unroll
        for (int i = 0; i < N; ++i)
            stg[i] = __builtin_bit_cast(uint4, *(const __attribute__((address_space(1))) u32x4*)(col + min(o.off[i], max_off)));
        w104 = *(const __attribute__((address_space(1))) uint32_t*)(col + min(o.off104, max104));
        xs0.load(T, valid ? b : 0);
        xs1.load(T, valid ? b + 1 : 1);
    }
    __device__ __forceinline__ void commit(uint8_t* slot) const {
        const int lane = kq_lane();
#pragma unroll
        for (int i = 0; i < N; ++i) reinterpret_cast<uint4*>(slot)[64 * i + lane] = stg[i];
        reinterpret_cast<uint32_t*>(slot + TR * ROWB)[lane & 31] = w104;     // lanes 32..63 repeat 0..31
        xs0.commit(slot + WSLOT);
        xs1.commit(slot + WSLOT + 1024 * NTOK);
    }
    static __device__ __forceinline__ void compute(const KqDesc& T, const uint8_t* slot, int tile, int b,
                                                   float (&acc)[NTOK]) {
        (void)T; (void)tile; (void)b;
        const int lane = kq_lane(), k = lane & 1, r = lane >> 1;
        const uint8_t* rowp = slot + r * ROWB + k * 208;
        const uint32_t w52 = k ? lds_read1(slot + TR * ROWB + 4 * r) : lds_read1(rowp + 208);
        q6_block_mac<NTOK>(rowp, w52, k ? 16u : 0u, slot + WSLOT + k * 1024 * NTOK, acc);
    }
};

// ------------------------------------------------------------ tile results
// Write a tile's row results: lane = row of a 64-row tile; of a 32-row tile
// the even lane of the pair that holds the row.
template <int NTOK, int TR>
__device__ __forceinline__ void write_rows(const KqDesc& T, int tile, const float (&v)[NTOK]) {
    const int lane = kq_lane();
    const int r = TR == kTileRows ? lane : lane >> 1;
    const int r0 = tile * TR;
    if ((TR == kTileRows || (lane & 1) == 0) && r < T.rows - r0) {
#pragma unroll
        for (int t = 0; t < NTOK; ++t) gfloat(T.y)[t * T.ldy + r0 + r] = v[t];
    }
}

// The workspace slot of a tile that several workgroups share.  Run v of
// the tensor starts at segment B_v = v*q + min(v, r) (q = seg_q, r = seg_r),
// and a tile is shared iff some B_v (1 <= v < P) falls strictly inside it.
// Runs shorter than a tile (q < nseg): the slot is the tile (the runs cover
// fewer segments than P * nseg, so there are fewer tiles than P).  Runs of
// a tile or more: a tile holds at most one boundary, and the slot is v - 1
// for the first boundary v after the tile's first segment.  Either way the
// workspace holds at most min(tiles, P - 1) slots of nseg segment sums,
// bounded by the grid and the row length, not by the number of rows.
__device__ __forceinline__ int shared_slot(const KqDesc& T, int tile) {
    const int q = T.seg_q, r = T.seg_r;
    if (q < T.nseg) return tile;
    const int t0 = tile * T.nseg;                   // segments before the tile
    return t0 < r * (q + 1) ? t0 / (q + 1) : (t0 - r) / q;
}

// Segment sum of a shared tile -> its workspace slot.  Partials and counters
// are only ever touched with device-scope atomic loads and stores, which the
// hardware keeps coherent across the XCDs' L2 caches (they carry the
// device-coherence bit), so no L2-wide writeback/invalidate is needed.
template <int NTOK>
__device__ __forceinline__ void store_partial(const KqDesc& T, int slot, int seg, const float (&v)[NTOK]) {
    const int lane = kq_lane();
    gfloat_t dst = gfloat(T.partials) + ((size_t)slot * T.nseg + seg) * (NTOK * kTileRows);
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
        __hip_atomic_store(dst + t * kTileRows + lane, v[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The segment sums of shared-tile slot `slot`, added in segment order
// (sum[t] starts at zero), for this lane's row of a 64-lane slot.
template <int NTOK>
__device__ __forceinline__ void sum_partials(const KqDesc& T, int slot, float (&sum)[NTOK]) {
    gfloat_t src = gfloat(T.partials) + (size_t)slot * T.nseg * (NTOK * kTileRows) + kq_lane();
#pragma unroll
    for (int t = 0; t < NTOK; ++t) sum[t] = 0.0f;
    // Batches of kFixBatch segment sums are requested together (indices past
    // the last segment re-read the last one and are not added), then added
    // in segment order: a 26-segment row of one token plane in one batch.
    constexpr int kFixBatch = NTOK == 1 ? 32 : NTOK == 2 ? 16 : 8;
    for (int p0 = 0; p0 < T.nseg; p0 += kFixBatch) {
        float v[kFixBatch][NTOK];
#pragma unroll
        for (int k = 0; k < kFixBatch; ++k) {
            const int p = min(p0 + k, T.nseg - 1);
#pragma unroll
            for (int t = 0; t < NTOK; ++t)
                v[k][t] = __hip_atomic_load(src + ((size_t)p * NTOK + t) * kTileRows, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        }
#pragma unroll
        for (int k = 0; k < kFixBatch; ++k) {
            if (p0 + k < T.nseg) {
#pragma unroll
                for (int t = 0; t < NTOK; ++t) sum[t] += v[k][t];
            }
        }
    }
}

// This workgroup stored `count` segment sums of a shared tile.  Ordering:
// the stores are complete (vmcnt drained) before the counter moves, and
// the last contributor reads the partials only after its increment
// returned; it adds all segment sums of the tile in order and resets the
// counter for the next launch.
template <int NTOK, int TR>
__device__ __forceinline__ void arrive(const KqDesc& T, int tile, int slot, int count) {
    const int lane = kq_lane();
    __attribute__((address_space(1))) uint32_t* ctr = (__attribute__((address_space(1))) uint32_t*)(T.counters + slot);
    uint32_t old = 0;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, (uint32_t)count, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (old + (uint32_t)count != (uint32_t)T.nseg) return;
    float sum[NTOK];
    sum_partials<NTOK>(T, slot, sum);
    write_rows<NTOK, TR>(T, tile, sum);
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- branch-free forms for the pipelined kernel.  Its loops must stay
// uniform: a lane-conditional block (if (lane == 0) ...) ahead of a loop's
// back edge lets the compiler split the loop so that lanes run different
// iterations, and a value shared through readfirstlane then comes from the
// wrong lane.  So every lane executes the same instructions: a flag store
// or a counter update that belongs to lane 0 is made by every lane, lane 0
// on the flag and lane i on a sink word of its own (no two lanes on one
// word, so no serialization); global stores and atomics that only some
// lanes may make go through buffer instructions whose out-of-range offset
// makes the hardware drop the other lanes.
constexpr uint32_t kBufDrop = 0x80000000u;      // a buffer offset past every range used here
typedef __attribute__((address_space(3))) volatile uint32_t* lsync_t;
typedef __attribute__((address_space(3))) uint32_t* lword_t;

// Lane 0's word w, the other lanes' sink words (sink[1..63]).
__device__ __forceinline__ lsync_t lane0_word(lsync_t w, lsync_t sink) {
    const int lane = kq_lane();
    return lane == 0 ? w : sink + lane;
}
// *w = v (lane 0), sink words for the rest.
__device__ __forceinline__ void lds_set(lsync_t w, lsync_t sink, uint32_t v) { *lane0_word(w, sink) = v; }
// Old value of an LDS counter that this wave moves by one (uniform).
__device__ __forceinline__ uint32_t lds_bump(lsync_t w, lsync_t sink) {
    const uint32_t old = __hip_atomic_fetch_add((lword_t)lane0_word(w, sink), kq_lane() == 0 ? 1u : 0u,
                                                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return __builtin_amdgcn_readfirstlane(old);
}

// write_rows for a 32-row tile: the even lane of each pair stores its row.
template <int NTOK>
__device__ __forceinline__ void write_rows_bf(const KqDesc& T, int tile, const float (&v)[NTOK]) {
    const int lane = kq_lane();
    const int r0 = tile * 32, rows_here = min(32, T.rows - r0), r = lane >> 1;
    const uint32_t off = ((lane & 1) == 0 && r < rows_here) ? 4u * (uint32_t)r : kBufDrop;
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
        const __amdgpu_buffer_rsrc_t y = __builtin_amdgcn_make_buffer_rsrc(T.y + t * T.ldy + r0, (short)0,
                                                                          4 * rows_here, kBufFlags);
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v[t]), y, off, 0, 0);
    }
}

// arrive(T, tile, slot, count) for a 32-row tile, branch-free.
template <int NTOK>
__device__ __forceinline__ void arrive_bf(const KqDesc& T, int tile, int slot, int count) {
    __attribute__((address_space(1))) uint32_t* ctr = (__attribute__((address_space(1))) uint32_t*)(T.counters + slot);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    const __amdgpu_buffer_rsrc_t c = __builtin_amdgcn_make_buffer_rsrc(T.counters + slot, (short)0, 4, kBufFlags);
    uint32_t old = (uint32_t)__builtin_amdgcn_raw_ptr_buffer_atomic_add_i32(count, c, kq_lane() == 0 ? 0u : kBufDrop, 0, 0);
    old = __builtin_amdgcn_readfirstlane(old);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (old + (uint32_t)count != (uint32_t)T.nseg) return;
    float sum[NTOK];
    sum_partials<NTOK>(T, slot, sum);
    write_rows_bf<NTOK>(T, tile, sum);
    __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);     // every lane: the same word
}

// A wave whose column arrives late gets the SIMD first: on a launch that
// lasts about as long as the memory system takes to deliver its bytes, the
// waves served last would otherwise share their SIMD's VALU with waves that
// are not on the critical path.  Ticks of the 100 MHz real-time counter
// since the run started: 3, 4.5 and 6 us raise the priority to 1, 2, 3 (a
// large matrix runs at 3 after its first columns, the same for every wave).
__device__ __forceinline__ void late_priority(uint64_t t_start) {
    const uint64_t dt = __builtin_amdgcn_s_memrealtime() - t_start;
    if (dt > 600) __builtin_amdgcn_s_setprio(3);
    else if (dt > 450) __builtin_amdgcn_s_setprio(2);
    else if (dt > 300) __builtin_amdgcn_s_setprio(1);
}

// ------------------------------------------------------------ a run of segments
// Segments j0..j1-1 of tensor T (tile-major), one super-block column at a
// time.  DEPTH columns are in flight in DEPTH register sets used in turn:
// the loads of column i+DEPTH go into the set of column i as soon as column
// i has been written to LDS, so a workgroup's first DEPTH columns are
// requested at once.  In 64-row tiles Q4_K and Q5_K use DEPTH 2, Q6_K 1
// (36, 44 and 64 staging registers a column); in 32-row tiles every format
// keeps one block-pair step in flight.
//
// The step is written out once per register set (static indices) and every
// step refills its set unconditionally (a column past the run reads a
// dummy address): a set whose loads may be in flight is then never merged
// with another value at a branch join, where the compiler would copy it and
// wait for the loads.
//
// Positions advance (tile, b) -> (tile, b+1) or (tile+1, 0) (b+2 in 32-row
// tiles, which take two blocks a step), carrying the segment index
// j = tile*nseg + b/S along (it moves on at a segment's last step or a
// row's end); a column whose segment is >= j1 lies past the end of the run.
// S is 1, 2 or 4 (4 only in 32-row tiles), smask = S - 1: a 64-row step ends
// its segment when (b & smask) == smask, a 32-row step when b + 2 is a
// multiple of S.  All of it is 32-bit scalar arithmetic (segment counts fit
// in int32).
#define KQ_LAST_OF_SEG(b_) (Col::CPS == 2 ? ((((b_) + 2) & smask) == 0) : (((b_) & smask) == smask))
#define KQ_ADVANCE(t_, b_, j_)                                      \
    {                                                               \
        if ((b_) + Col::CPS >= nb) { ++(t_); (b_) = 0; ++(j_); }      \
        else { (j_) += KQ_LAST_OF_SEG(b_) ? 1 : 0; (b_) += Col::CPS; } \
    }
#define KQ_STEP(k_)                                                                            \
    {                                                                                          \
        __syncthreads();                                /* earlier reads of the slot done */   \
        c[k_].commit(slot);                                                                    \
        late_priority(t_start);                                                                \
        {                                                                                      \
            const bool valid = ij < j1;                                                        \
            c[k_].stage(T, offs, itile, ib, valid);                                            \
            if (valid) KQ_ADVANCE(itile, ib, ij)                                               \
        }                                                                                      \
        const bool row_end = b + Col::CPS >= nb;                                               \
        const bool seg_end = row_end || KQ_LAST_OF_SEG(b);                                     \
        const int ntile = row_end ? tile + 1 : tile;                                           \
        const int nbb = row_end ? 0 : b + Col::CPS;                                            \
        const int nj = seg_end ? j + 1 : j;                                                    \
        const bool has_next = nj < j1;                                                         \
        __syncthreads();                                /* slot written */                     \
        Col::compute(T, slot, tile, b, acc);                                                   \
        if (seg_end) {                                                                         \
            if constexpr (Col::TR != kTileRows) {       /* the pair's two blocks */            \
                _Pragma("unroll") for (int t = 0; t < NTOK; ++t) acc[t] = acc[t] + dpp_xor1(acc[t]); \
            }                                                                                  \
            if (owned) {                                                                       \
                _Pragma("unroll") for (int t = 0; t < NTOK; ++t) tsum[t] = tsum[t] + acc[t];   \
            } else {                                                                           \
                store_partial<NTOK>(T, wslot, seg, acc);                                       \
                ++pending;                                                                     \
            }                                                                                  \
            _Pragma("unroll") for (int t = 0; t < NTOK; ++t) acc[t] = 0.0f;                    \
            if (row_end || !has_next) {                                                        \
                if (owned) {                                                                   \
                    write_rows<NTOK, Col::TR>(T, tile, tsum);                                  \
                    _Pragma("unroll") for (int t = 0; t < NTOK; ++t) tsum[t] = 0.0f;           \
                } else {                                                                       \
                    arrive<NTOK, Col::TR>(T, tile, wslot, pending);                            \
                    pending = 0;                                                               \
                }                                                                              \
            }                                                                                  \
            seg = row_end ? 0 : seg + 1;                                                       \
        }                                                                                      \
        if (!has_next) break;                                                                  \
        if (row_end) {                                                                         \
            owned = nj + nseg <= j1;                                                           \
            if (!owned) wslot = shared_slot(T, ntile);                                         \
        }                                                                                      \
        tile = ntile;                                                                          \
        b = nbb;                                                                               \
        j = nj;                                                                                \
    }

template <class Col, int NTOK, int DEPTH>
__device__ __forceinline__ void run_segments(const KqDesc& T, int j0, int j1, uint8_t* slot) {
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    static_assert(DEPTH >= 1 && DEPTH <= 3, "1..3 register sets");
    const int nseg = T.nseg, nb = T.nb, smask = T.seg - 1;
    int tile = j0 / nseg;
    int seg = j0 - tile * nseg;
    int b = seg * T.seg;
    int j = j0;
    typename Col::Offsets offs;
    offs.init(T);
    float acc[NTOK], tsum[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) { acc[t] = 0.0f; tsum[t] = 0.0f; }
    int pending = 0;
    bool owned = seg == 0 && j0 + nseg <= j1;
    int wslot = owned ? 0 : shared_slot(T, tile);     // workspace slot of a shared tile
    Col c[DEPTH];
    int itile = tile, ib = b, ij = j;     // the next column to request
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
        const bool valid = ij < j1;
        c[d].stage(T, offs, itile, ib, valid);
        if (valid) KQ_ADVANCE(itile, ib, ij)
    }
#pragma unroll 1
    while (true) {
        KQ_STEP(0)
        if constexpr (DEPTH > 1) KQ_STEP(1)
        if constexpr (DEPTH > 2) KQ_STEP(2)
    }
}
#undef KQ_STEP
#undef KQ_ADVANCE
#undef KQ_LAST_OF_SEG

// ------------------------------------------------------------ the kernel
#ifndef KQ_DEPTH_Q4
#define KQ_DEPTH_Q4 2
#endif
#ifndef KQ_DEPTH_Q5
#define KQ_DEPTH_Q5 2
#endif
#ifndef KQ_DEPTH_Q6
#define KQ_DEPTH_Q6 1
#endif
constexpr int kDepthQ4 = KQ_DEPTH_Q4, kDepthQ5 = KQ_DEPTH_Q5;
// (two Q6_K columns in flight fit the register file only for one token
// plane, and measured no faster than one)
template <int NTOK> constexpr int kDepthQ6 = NTOK == 1 ? KQ_DEPTH_Q6 : 1;

// Workgroup w belongs to the tensor i with wg_end[i-1] <= w < wg_end[i] and
// streams run u = w - wg_base of it: segments [u*seg_q + min(u, seg_r), ...).
template <int NTOK>
__global__ __launch_bounds__(64, 2) void kq_matvec_kernel(const KqLaunch L) {
    extern __shared__ uint4 kq_slot[];
    uint8_t* slot = reinterpret_cast<uint8_t*>(kq_slot);
    // the head, in one batch of scalar loads (it carries the grid size, so
    // the workgroup's index needs no other kernel-argument load)
    const u32x8* hp = reinterpret_cast<const u32x8*>(&L.h);
    const u32x8 g0 = hp[0], g1 = hp[1], g2 = hp[2];
    asm volatile("" : : "s"(g0), "s"(g1), "s"(g2));
    const int n = (int)g0[0];
    const int w = xcd_remap(blockIdx.x, (int)g0[1]);
    // the tensor: count the tensors ending at or before w (the ends are
    // increasing; unused entries are INT32_MAX)
    int i = 0;
#pragma unroll
    for (int k = 0; k < kMaxSet; ++k) i += (int)(k < 8 ? g1[k] : g2[k - 8]) <= w ? 1 : 0;
    if (i >= n) return;
    const KqDesc T = load_uniform(L.t[i]);
    const int u = w - T.wg_base;
    const int j0 = u * T.seg_q + min(u, T.seg_r);
    const int j1 = j0 + T.seg_q + (u < T.seg_r ? 1 : 0);
    // 32-row tiles are planned for one and two token planes only
    if constexpr (NTOK <= 2) {
        // 32-row tiles keep one block-pair step in flight: with two, a
        // decode set and the large matrices both ran 1-8% slower (at two
        // waves a SIMD one step already keeps enough bytes in flight, and
        // the second register set only adds pressure)
        constexpr int DP = 1;
        if (T.tile_rows != kTileRows) {
            switch (T.fmt) {
            case KQ_Q4_K: run_segments<K45Pair<KQ_Q4_K, NTOK>, NTOK, DP>(T, j0, j1, slot); break;
            case KQ_Q5_K: run_segments<K45Pair<KQ_Q5_K, NTOK>, NTOK, DP>(T, j0, j1, slot); break;
            default: run_segments<Q6Pair<NTOK>, NTOK, DP>(T, j0, j1, slot); break;
            }
            return;
        }
    }
    switch (T.fmt) {
    case KQ_Q4_K: run_segments<K45Column<KQ_Q4_K, NTOK>, NTOK, kDepthQ4>(T, j0, j1, slot); break;
    case KQ_Q5_K: run_segments<K45Column<KQ_Q5_K, NTOK>, NTOK, kDepthQ5>(T, j0, j1, slot); break;
    default:
        if (T.nb & 1) run_segments<Q6Column<NTOK, true>, NTOK, kDepthQ6<NTOK>>(T, j0, j1, slot);
        else run_segments<Q6Column<NTOK, false>, NTOK, kDepthQ6<NTOK>>(T, j0, j1, slot);
        break;
    }
}

// ------------------------------------------------------------ the pipelined kernel
// Launches whose tensors all run in 32-row tiles with two-block segments
// (every decode set and every large matrix at one token plane, at two up to
// 16384 rows), with at least four steps a compute unit, and whose x fits in
// LDS beside a ring of at least eight steps take this kernel: one workgroup
// a compute unit, holding two kinds of waves.
//   * The producer (kPcProducers: one wave) only moves bytes.  It issues the
//     direct buffer -> LDS loads of the run's steps, in order, into a ring of
//     LDS slots, keeps four steps in flight, waits for the oldest with vmcnt
//     and publishes its slot.
//   * Consumers (kPcConsumers: 12; with the producer at most four waves a
//     SIMD, within the kernel's 128 registers) only compute.  A free consumer claims the
//     next position of the workgroup's run (an LDS counter), waits for its
//     slot, copies its lane's block into registers, frees the slot and
//     computes the step exactly as kq_matvec_kernel does.  Claiming in
//     order, rather than a fixed share per consumer, frees each slot as soon
//     as any consumer is idle.
// x is resident: every x block the run reads, loaded once at the start by
// the consumers.
// So no wave waits to issue a load while it holds data to compute, and the
// run's bytes are requested as fast as the ring frees.  Position n of the
// run is segment j0 + n (one step: 32 rows x 2 blocks) in slot n % R.  The
// pair-added segment sum goes to its tile: a tile whose segments all lie in
// the run is folded in LDS, in segment order, by the consumer whose delivery
// completes it; a tile shared with other workgroups goes through the
// workspace exactly as in kq_matvec_kernel, so the bits are those of
// kq_matvec_kernel for the same plan.
// Deadlock freedom: positions are claimed in order; a consumer frees its
// slot before delivering, and waits only for the tile-fold slot it
// delivers to (until the tile TS places earlier is folded, which needs only
// lower positions), so the lowest undelivered position can always go on.
// Every wait is bounded: a broken handshake ends the wave (wrong results),
// it never hangs the GPU.
constexpr int kPcProducers = 1, kPcConsumers = 12, kPcWaves = kPcProducers + kPcConsumers;
constexpr int kPcSpin = 1 << 22;

// s_waitcnt for vmcnt <= N (expcnt and lgkmcnt not waited for)
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt has six bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0) (vmcnt and expcnt not waited for)
__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }

// Waits until *f == v, at most kPcSpin polls; false on time-out.  The
// polled word goes through readfirstlane so that the test is a scalar one:
// every loop around a wait is then uniform to the compiler, which otherwise
// may lower it as a divergent loop and run lanes in different iterations
// (the claim in pc_consume relies on lane 0 being in every iteration).
__device__ __forceinline__ bool spin_until(lsync_t f, uint32_t v) {
    for (int k = 0; k < kPcSpin; ++k) {
        if ((uint32_t)__builtin_amdgcn_readfirstlane(*f) == v) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// The LDS of one workgroup for tensor T.  Dynamic (offsets in bytes): R
// weight slots of W bytes; x, one X-byte slot per segment of a tile row
// (slot s holds blocks 2s and 2s + 1); then the fold slots' segment sums
// [TS][nseg][NTOK][32] floats.  Static (kq_pc_sync, words): ready[R]
// (position + 1 once its weights are in), wdone[R] (position + 1 once its
// weights are read into registers), owner[TS] and count[TS] of the fold
// slots, the claim counter, the consumers that have loaded their share of x,
// and 64 sink words (lane0_word).  The flags live in an array of their own,
// apart from the slots the direct loads write, so polling them needs no
// wait for the loads in flight.
constexpr int kPcMaxSlots = 16, kPcMaxFold = 16;
struct PcLayout {
    int R, TS, W, X, xs, sums;
    bool nt;        // non-temporal weight loads
    __device__ __forceinline__ PcLayout(const KqDesc& T, int w, int x) {
        R = T.reserved0 & 255;
        TS = (T.reserved0 >> 8) & 255;
        nt = (T.reserved0 >> 16) & 1;
        W = w;
        X = x;
        xs = R * W;
        sums = xs + T.nseg * X;
    }
    static constexpr int ready = 0, wdone = kPcMaxSlots, owner = 2 * kPcMaxSlots, count = owner + kPcMaxFold,
                         claim = count + kPcMaxFold, xready = claim + 1, sink = xready + 1, words = sink + 64;
};

// Steps the producer keeps in flight: four (D * LOADS <= 63 for vmcnt).  One
// producer issuing its steps in order, four deep, with non-temporal loads on
// small launches, against two producers on alternate steps two deep each
// with ordinary loads: a decode set 15.0 -> 14.6 us, 16 rotating sets 14.0
// -> 13.5 us, the 202,048-row matrices unchanged.  Two producers gained
// nothing from the non-temporal hint (a decode set 15.33 us either way).
template <class Col>
constexpr int pc_depth() { return 63 / Col::LOADS < 4 ? 63 / Col::LOADS : 4; }

// The pipelined kernel needs a ring of at least this many step slots: the
// 19,968-column FFN down, whose resident x leaves room for six Q4_K steps,
// ran 8% slower in it than in the one-wave kernel (27.1 against 25.0 us).
constexpr int kPcMinSlots = 8;

// The steps of one producer: positions p, p + kPcProducers, ... of the run.
// Before issuing position n it waits until position n - R has left its
// slot (R is a multiple of kPcProducers of at least kPcProducers * D, so
// that position is its own and already published).
template <class Col, int NTOK>
__device__ __forceinline__ void pc_produce(const KqDesc& T, int j0, int nsteps, uint8_t* lds, lsync_t sync,
                                           const PcLayout& Y, int p) {
    constexpr int LD = Col::LOADS, D = pc_depth<Col>();
    static_assert(D >= 2, "two steps in flight");
    typename Col::Offsets offs;
    offs.init(T);
    const int nseg = T.nseg;
    int issued = 0, published = 0;
    for (int n = p; n < nsteps; n += kPcProducers) {
        const int ws = n % Y.R;
        if (n >= Y.R && !spin_until(sync + PcLayout::wdone + ws, (uint32_t)(n - Y.R + 1))) return;
        const int j = j0 + n, tile = j / nseg, b = 2 * (j - tile * nseg);
        if (Y.nt) Col::template dma_w<kNonTemporal>(T, offs, tile, b, lds + ws * Y.W);
        else Col::template dma_w<0>(T, offs, tile, b, lds + ws * Y.W);
        ++issued;
        // a step is published with D steps in flight: the first D steps go
        // out back to back before any wait (publishing the first step as
        // soon as the second was issued held the third and fourth back until
        // the first had landed: the 202,048-row Q6_K 197.6 -> 193.0 us, the
        // FFN gate + up 39.0 -> 37.7 us, the attention output 10.64 ->
        // 10.12 us, 16 rotating decode sets 13.59 -> 13.28 us; the 52-layer
        // stream 14.67 -> 14.76 us)
        if (issued - published == D) {
            wait_vm<(D - 1) * LD>();
            const int pos = p + kPcProducers * published;
            lds_set(sync + PcLayout::ready + pos % Y.R, sync + PcLayout::sink, (uint32_t)(pos + 1));
            ++published;
        }
    }
    while (published < issued) {
        const int left = issued - published - 1;       // steps that may stay in flight
        if (left >= 3) wait_vm<3 * LD>();
        else if (left == 2) wait_vm<2 * LD>();
        else if (left == 1) wait_vm<LD>();
        else wait_vm<0>();
        const int pos = p + kPcProducers * published;
        lds_set(sync + PcLayout::ready + pos % Y.R, sync + PcLayout::sink, (uint32_t)(pos + 1));
        ++published;
    }
}

// One consumer (c = 0 .. kPcConsumers - 1): first its share of x (pieces
// c, c + kPcConsumers, ... of 1 KB: one token plane of one block of the
// segments the run reads, segment s in slot s % nseg), then positions
// claimed in order until the run is done.
template <class Col, int NTOK>
__device__ __forceinline__ void pc_consume(const KqDesc& T, int j0, int j1, uint8_t* lds, lsync_t sync,
                                           const PcLayout& Y, int c) {
    const uint64_t t_start = __builtin_amdgcn_s_memrealtime();
    const int lane = kq_lane();
    const int nseg = T.nseg, nsteps = j1 - j0;
    const int first_owned = (j0 + nseg - 1) / nseg;     // first tile that lies wholly in the run
    {
        const int need = min(nsteps, nseg), seg0 = j0 % nseg;
        for (int q = c; q < need * 2 * NTOK; q += kPcConsumers) {
            const int k = q / (2 * NTOK), part = q - k * 2 * NTOK, kb = part / NTOK, t = part - kb * NTOK;
            const int sg = seg0 + k < nseg ? seg0 + k : seg0 + k - nseg;
            kq::dma16(gbytes(T.x) + 4 * (t * T.ldx + 256 * (2 * sg + kb) + 4 * lane),
                        lds + Y.xs + sg * Y.X + 1024 * part);
        }
        wait_vm<0>();
        (void)lds_bump(sync + PcLayout::xready, sync + PcLayout::sink);
        if (!spin_until(sync + PcLayout::xready, (uint32_t)kPcConsumers)) return;
    }
    for (;;) {
        const int n = (int)lds_bump(sync + PcLayout::claim, sync + PcLayout::sink);
        if (n >= nsteps) break;
        const int ws = n % Y.R;
        if (!spin_until(sync + PcLayout::ready + ws, (uint32_t)(n + 1))) return;
        const int j = j0 + n, tile = j / nseg, seg = j - tile * nseg;
        typename Col::Regs regs;
        Col::load_regs(lds + ws * Y.W, regs);
        wait_lds();                                      // the block is in registers
        lds_set(sync + PcLayout::wdone + ws, sync + PcLayout::sink, (uint32_t)(n + 1));
        late_priority(t_start);
        float acc[NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) acc[t] = 0.0f;
        Col::compute_regs(regs, lds + Y.xs + seg * Y.X, acc);
#pragma unroll
        for (int t = 0; t < NTOK; ++t) acc[t] = acc[t] + dpp_xor1(acc[t]);     // the pair's two blocks
        if (tile * nseg >= j0 && (tile + 1) * nseg <= j1) {
            // a tile of this run: fold slot (tile - first_owned) % TS, free once
            // the tile TS places earlier has been folded
            const int ts = (tile - first_owned) % Y.TS;
            if (!spin_until(sync + PcLayout::owner + ts, (uint32_t)tile)) return;
            float* sums = reinterpret_cast<float*>(lds + Y.sums) + ts * nseg * NTOK * 32;    // [TS][nseg][NTOK][32]
            // both lanes of a pair hold the pair sum: each stores it
#pragma unroll
            for (int t = 0; t < NTOK; ++t) sums[(seg * NTOK + t) * 32 + (lane >> 1)] = acc[t];
            wait_lds();
            if (lds_bump(sync + PcLayout::count + ts, sync + PcLayout::sink) == (uint32_t)(nseg - 1)) {
                float sum[NTOK];
#pragma unroll
                for (int t = 0; t < NTOK; ++t) sum[t] = 0.0f;
                for (int s2 = 0; s2 < nseg; ++s2) {
#pragma unroll
                    for (int t = 0; t < NTOK; ++t) sum[t] = sum[t] + sums[(s2 * NTOK + t) * 32 + (lane >> 1)];
                }
                write_rows_bf<NTOK>(T, tile, sum);
                wait_lds();
                lds_set(sync + PcLayout::count + ts, sync + PcLayout::sink, 0u);
                lds_set(sync + PcLayout::owner + ts, sync + PcLayout::sink, (uint32_t)(tile + Y.TS));
            }
        } else {
            // a tile shared with other workgroups: straight to the workspace
            // (the round trips of different segments overlap)
            const int wslot = shared_slot(T, tile);
            store_partial<NTOK>(T, wslot, seg, acc);
            arrive_bf<NTOK>(T, tile, wslot, 1);
        }
    }
}

template <class Col, int NTOK>
__device__ __forceinline__ void pc_run(const KqDesc& T, int j0, int j1, uint8_t* lds, lsync_t sync, int wave) {
    const PcLayout Y(T, Col::PC_W, Col::PC_X);
    // flags zero, fold slots owned by the run's first TS whole tiles
    const int first_owned = (j0 + T.nseg - 1) / T.nseg;
    for (int k = threadIdx.x; k < 2 * kPcMaxSlots; k += blockDim.x) sync[k] = 0u;
    for (int k = threadIdx.x; k < kPcMaxFold; k += blockDim.x) {
        sync[PcLayout::owner + k] = (uint32_t)(first_owned + k);
        sync[PcLayout::count + k] = 0u;
    }
    if (threadIdx.x == 0) {
        sync[PcLayout::claim] = 0u;
        sync[PcLayout::xready] = 0u;
    }
    __syncthreads();
    if (wave < kPcProducers) {
        __builtin_amdgcn_s_setprio(3);
        pc_produce<Col, NTOK>(T, j0, j1 - j0, lds, sync, Y, wave);
    } else {
        pc_consume<Col, NTOK>(T, j0, j1, lds, sync, Y, wave - kPcProducers);
    }
}

template <int NTOK>
__global__ __launch_bounds__(64 * kPcWaves, 1) void kq_pc_kernel(const KqLaunch L) {
    extern __shared__ uint4 kq_pc_lds[];
    __shared__ uint32_t kq_pc_sync[PcLayout::words];
    uint8_t* lds = reinterpret_cast<uint8_t*>(kq_pc_lds);
    const lsync_t sync = (lsync_t)(kq_pc_sync);
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));    // uniform: scalar bookkeeping
    const u32x8* hp = reinterpret_cast<const u32x8*>(&L.h);
    const u32x8 g0 = hp[0], g1 = hp[1], g2 = hp[2];
    asm volatile("" : : "s"(g0), "s"(g1), "s"(g2));
    const int n = (int)g0[0];
    const int w = xcd_remap(blockIdx.x, (int)g0[1]);
    int i = 0;
#pragma unroll
    for (int k = 0; k < kMaxSet; ++k) i += (int)(k < 8 ? g1[k] : g2[k - 8]) <= w ? 1 : 0;
    if (i >= n) return;
    const KqDesc T = load_uniform(L.t[i]);
    const int u = w - T.wg_base;
    const int j0 = u * T.seg_q + min(u, T.seg_r);
    const int j1 = j0 + T.seg_q + (u < T.seg_r ? 1 : 0);
    switch (T.fmt) {
    case KQ_Q4_K: pc_run<K45Pair<KQ_Q4_K, NTOK>, NTOK>(T, j0, j1, lds, sync, wave); break;
    case KQ_Q5_K: pc_run<K45Pair<KQ_Q5_K, NTOK>, NTOK>(T, j0, j1, lds, sync, wave); break;
    default: pc_run<Q6Pair<NTOK>, NTOK>(T, j0, j1, lds, sync, wave); break;
    }
}

// The pipelined kernel's sizes for a tensor of this format at ntok (1 or
// 2): LDS bytes of a step's weights (*w) and of a segment's x (*x), and the
// steps a producer keeps in flight (*d).
template <class Col>
static void pc_sizes_t(int* w, int* x, int* d) {
    *w = Col::PC_W;
    *x = Col::PC_X;
    *d = pc_depth<Col>();
}
void pc_sizes(int32_t fmt, int32_t ntok, int* w, int* x, int* d) {
    if (ntok == 1) {
        if (fmt == KQ_Q4_K) pc_sizes_t<K45Pair<KQ_Q4_K, 1>>(w, x, d);
        else if (fmt == KQ_Q5_K) pc_sizes_t<K45Pair<KQ_Q5_K, 1>>(w, x, d);
        else pc_sizes_t<Q6Pair<1>>(w, x, d);
    } else {
        if (fmt == KQ_Q4_K) pc_sizes_t<K45Pair<KQ_Q4_K, 2>>(w, x, d);
        else if (fmt == KQ_Q5_K) pc_sizes_t<K45Pair<KQ_Q5_K, 2>>(w, x, d);
        else pc_sizes_t<Q6Pair<2>>(w, x, d);
    }
}

// ------------------------------------------------------------ embedding rows
// The embedding lookup (muser-book Ch 6 section 6.7): out[t][j] is element j
// of row ids[t] of a Q4_K table, dequantized.  A wave takes one block of one
// row; lane l forms elements 4l..4l+3, which share a sub-block and a qs word
// (low nibbles for the first 8 lanes of each 16, high for the next 8), and
// stores them as one 16-byte write, so a wave writes the block's 1 KB
// contiguously.  Four waves a workgroup take four consecutive blocks.
// d*sc and dmin*m are exact in float32, and so is (d*sc)*q; the difference
// is rounded once, so every value is the exact weight correctly rounded.
__global__ __launch_bounds__(256) void kq_embed_kernel(const uint8_t* table, int64_t rows, int32_t nb,
                                                        int32_t groups, const int32_t* ids, float* out,
                                                        int64_t ldo) {
    const int t = blockIdx.x / groups;
    const int b = (blockIdx.x - t * groups) * 4 + (int)(threadIdx.x >> 6);
    if (b >= nb) return;
    const int lane = threadIdx.x & 63;
    const int64_t id = ids[t];
    float4 v;
    if (id < 0 || id >= rows) {
        v = make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""));
    } else {
        const uint8_t* blk = table + (id * nb + b) * 144;
        const uint4 hdr = *reinterpret_cast<const uint4*>(blk);
        const int g = lane >> 4, hi = (lane >> 3) & 1, j = 2 * g + hi;
        const uint32_t word = *reinterpret_cast<const uint32_t*>(blk + 16 + 4 * (8 * g + (lane & 7)));
        const uint32_t q = (word >> (4 * hi)) & 0x0F0F0F0Fu;
        const K4Scales S = k4_scales(hdr.y, hdr.z, hdr.w);
        const float dsc = f16_to_f32(hdr.x & 0xFFFFu) * (float)k4_sc(S, j);     // exact
        const float dm = f16_to_f32(hdr.x >> 16) * (float)k4_m(S, j);           // exact
        v.x = dsc * (float)(q & 0xFF) - dm;
        v.y = dsc * (float)((q >> 8) & 0xFF) - dm;
        v.z = dsc * (float)((q >> 16) & 0xFF) - dm;
        v.w = dsc * (float)(q >> 24) - dm;
    }
    reinterpret_cast<float4*>(out + (int64_t)t * ldo + 256 * b)[lane] = v;
}

int launch_embed(const uint8_t* table, int64_t rows, int64_t cols, const int32_t* ids, int32_t n, float* out,
                 int64_t ldo, hipStream_t stream) {
    const int32_t nb = (int32_t)(cols / 256);
    const int32_t groups = (nb + 3) / 4;
    hipLaunchKernelGGL(kq_embed_kernel, dim3((unsigned)(n * groups)), dim3(256), 0, stream, table, rows, nb, groups,
                       ids, out, ldo);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

// ------------------------------------------------------------ many token planes on the bf16 matrix cores
// Q4_K / Q5_K: the same product for many token planes with v_mfma_f32_16x16x32_bf16 (16
// times the float32 matrix rate), the operands kept exact enough for the
// per-row bound (muser-book Ch 6 Figure 6.7 puts prefill on half-precision
// matrix products; here the half-precision operands are exact):
// - each sub-block's codes are offset by an integer c = round(dmin*m /
//   (d*sc)) clamped to the code range, so W = a*(q - c) - b' with a = d*sc,
//   b' = dmin*m - a*c (one rounding) and |b'| <= |a|/2 where cancellation
//   can happen; q - c is a small integer, exact in bf16;
// - x is split into two bf16 parts, hi = bf16(x) and lo = bf16(x - hi), so
//   hi + lo is x to 2^-18 relative;
// - per sub-block j and token, C_j = sum (q - c)*(hi + lo) comes from two
//   bf16 products (codes against each part); X_j, the sub-block's sum of x,
//   is summed in float32 when x is staged;
// - a block adds sum_j a_j*C_j - sum_j b'_j*X_j into the row, the second
//   sum over the eight sub-blocks as two float32 products.
// Every error term is then relative to |W_e x_e| (|a*(q - c)| <= 2|W_e| and
// |b'| <= |W_e| for every element, as the rounding-to-nearest of c gives).
// Layout: a workgroup of NW waves takes NW/KS 16-row tiles and 16*TT
// tokens, a tile's blocks dealt over KS waves in turn.  In the products A
// is x (16 tokens x 32 elements of a sub-block) and B the codes (32
// elements x 16 rows): lane l supplies token l % 16 and row l % 16 over
// elements 8*(l/16) .. +7 of the sub-block, and ends with C for tokens
// 4*(l/16) + v of its own row l % 16, so the row's coefficients scale the
// lane's own results.  Each block's x (16*TT tokens) is split once by the
// workgroup into two bf16 planes in LDS, with its sub-block sums.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kMbRow = 528;                  // LDS bytes a token row of one bf16 plane (512 + 16)

// The two bf16 parts of four x values (each pair packed low element first).
__device__ __forceinline__ void split_x(const float4 v, uint2& hi, uint2& lo) {
    const bf16x2_t h01 = __builtin_convertvector((f32x2_t){v.x, v.y}, bf16x2_t);
    const bf16x2_t h23 = __builtin_convertvector((f32x2_t){v.z, v.w}, bf16x2_t);
    const f32x2_t b01 = __builtin_convertvector(h01, f32x2_t), b23 = __builtin_convertvector(h23, f32x2_t);
    const bf16x2_t l01 = __builtin_convertvector((f32x2_t){v.x - b01.x, v.y - b01.y}, bf16x2_t);
    const bf16x2_t l23 = __builtin_convertvector((f32x2_t){v.z - b23.x, v.w - b23.y}, bf16x2_t);
    hi = make_uint2(__builtin_bit_cast(uint32_t, h01), __builtin_bit_cast(uint32_t, h23));
    lo = make_uint2(__builtin_bit_cast(uint32_t, l01), __builtin_bit_cast(uint32_t, l23));
}

// Four codes (bytes of w, each 0..31) minus cf, as bf16 pairs (exact).
__device__ __forceinline__ uint2 codes_bf16(uint32_t w, float cf) {
    const f32x2_t a = {(float)(w & 0xFFu) - cf, (float)((w >> 8) & 0xFFu) - cf};
    const f32x2_t b = {(float)((w >> 16) & 0xFFu) - cf, (float)(w >> 24) - cf};
    return make_uint2(__builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2_t)),
                      __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2_t)));
}

template <int FMT, int TT, int KS, int NW>
__global__ __launch_bounds__(64 * NW) void kq_mmb_kernel(const uint8_t* w, int64_t row_bytes, int32_t rows, int32_t nb,
                                                     const float* x, int64_t ldx, int32_t ntok, float* y,
                                                     int64_t ldy) {
    static_assert(FMT == KQ_Q4_K || FMT == KQ_Q5_K, "Q4_K and Q5_K");
    static_assert(KS == 1 || KS == 2 || KS == 4, "1, 2 or 4 waves a tile");
    static_assert(NW == 4 || NW == 8, "four or eight waves a workgroup");
    constexpr int BB = FMT == KQ_Q4_K ? 144 : 176;
    constexpr int QS = FMT == KQ_Q4_K ? 16 : 48;      // byte offset of qs
    constexpr float QMAX = FMT == KQ_Q4_K ? 15.0f : 31.0f;
    constexpr int kTok = 16 * TT;
    constexpr int kXP = 16 * TT / NW;                  // float4 pieces of x a thread stages per block
    constexpr int kXR = kXP * KS;                      // ... per step (KS blocks)
    constexpr int kPlane = kTok * kMbRow;              // LDS bytes of one block's x, one part
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][KS * kPlane];
    __shared__ __attribute__((aligned(16))) float xsum[KS][8 * kTok];   // [sub-block][token] sums of x
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, h = lane >> 4;
    const int ks = wave % KS;                          // this wave's block of each step
    const int row0 = (blockIdx.x * (NW / KS) + wave / KS) * 16;
    const int tok0 = blockIdx.y * kTok;
    const int steps = (nb + KS - 1) / KS;
    // rows past the matrix repeat its last row; their results are not written
    const uint8_t* arow = w + (int64_t)min(row0 + r16, rows - 1) * row_bytes;
    // staging: thread tid moves float4 tid % 64 of tokens tid/64 + NW*i, i <
    // kXP, of each of the step's KS blocks (tokens past ntok repeat the last
    // plane, blocks past nb the last block; neither result is used)
    const float* xcol = x + 4 * (tid & 63);
    const int xtok = tok0 + (tid >> 6);
    float acc[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = 0.0f;
    u32x4 xr[kXR];
    uint4 hdr;
    uint32_t q[8], hb[2];
    // every step loads the next step's blocks unconditionally (past the
    // last step it loads the last one again, unused)
    auto load = [&](int st) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int64_t xb = 256 * (int64_t)min(st * KS + k, nb - 1);
#pragma unroll
            for (int i = 0; i < kXP; ++i)
                xr[k * kXP + i] =
                    *reinterpret_cast<const u32x4*>(xcol + (int64_t)min(xtok + NW * i, ntok - 1) * ldx + xb);
        }
        const int64_t bo = (int64_t)min(st * KS + ks, nb - 1) * BB;
        hdr = *reinterpret_cast<const uint4*>(arow + bo);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const uint2 v = *reinterpret_cast<const uint2*>(arow + bo + QS + 32 * g + 8 * h);
            q[2 * g] = v.x;
            q[2 * g + 1] = v.y;
        }
        if constexpr (FMT == KQ_Q5_K) {
            const uint2 v = *reinterpret_cast<const uint2*>(arow + bo + 16 + 8 * h);
            hb[0] = v.x;
            hb[1] = v.y;
        }
    };
    load(0);
    for (int st = 0; st < steps; ++st) {
        __syncthreads();                                    // the previous step's LDS reads are done
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int i = 0; i < kXP; ++i) {
                uint2 hi, lo;
                const float4 xv = __builtin_bit_cast(float4, xr[k * kXP + i]);
                split_x(xv, hi, lo);
                const int off = k * kPlane + ((tid >> 6) + NW * i) * kMbRow + 8 * (tid & 63);
                *reinterpret_cast<uint2*>(xs[0] + off) = hi;
                *reinterpret_cast<uint2*>(xs[1] + off) = lo;
                // the sub-block's sum of x: four elements here, then over the
                // eight lanes of the sub-block (lane pairs, quads, half rows)
                float s4 = (xv.x + xv.y) + (xv.z + xv.w);
                s4 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s4), 0xB1, 0xF, 0xF, false));
                s4 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s4), 0x4E, 0xF, 0xF, false));
                s4 += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, s4), 0x141, 0xF, 0xF, false));
                if ((tid & 7) == 0) xsum[k][((tid & 63) >> 3) * kTok + (tid >> 6) + NW * i] = s4;
            }
        const uint4 hd = hdr;
        uint32_t qq[8], hh[2];
#pragma unroll
        for (int i = 0; i < 8; ++i) qq[i] = q[i];
        hh[0] = hb[0];
        hh[1] = hb[1];
        __syncthreads();                                    // x of the step's blocks is in LDS
        load(min(st + 1, steps - 1));
        asm volatile("" : : : "memory");
        if (st * KS + ks >= nb) continue;                   // a ragged last step (the wave's own block)
        const uint8_t* xh_base = xs[0] + ks * kPlane;
        const uint8_t* xl_base = xs[1] + ks * kPlane;
        const float d = f16_to_f32(hd.x & 0xFFFFu), dmin = f16_to_f32(hd.x >> 16);
        const K4Scales S = k4_scales(hd.y, hd.z, hd.w);
        // sub-block coefficients: lane h of a row forms those of sub-blocks
        // 2h and 2h + 1; the row's other lanes take them by lane permute
        float ca[2], cc[2], cn[2];
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) {
            const int sh8 = 8 * (2 * (h & 1) + jj);
            const uint32_t scw = h < 2 ? S.sc_lo : S.sc_hi, mw = h < 2 ? S.m_lo : S.m_hi;
            const float a = d * (float)((scw >> sh8) & 0xFFu);            // exact
            const float bm = dmin * (float)((mw >> sh8) & 0xFFu);         // exact
            cc[jj] = __builtin_fminf(__builtin_fmaxf(__builtin_rintf(bm * __builtin_amdgcn_rcpf(a)), 0.0f), QMAX);
            cn[jj] = __builtin_fmaf(a, cc[jj], -bm);                      // -(b - a*c), one rounding
            ca[jj] = a;
        }
        // the offset terms sum_j -b'_j * X_j of the block, for every row and
        // token of the tile, as two float32 products over the sub-blocks:
        // lane group h brings sub-blocks 2h (first) and 2h + 1 (second),
        // whose -b' it formed itself
        float blk[TT][4];
#pragma unroll
        for (int t = 0; t < TT; ++t) {
            f32x4 O = {0.0f, 0.0f, 0.0f, 0.0f};
            O = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[ks][(2 * h) * kTok + 16 * t + r16], cn[0], O, 0, 0, 0);
            O = __builtin_amdgcn_mfma_f32_16x16x4f32(xsum[ks][(2 * h + 1) * kTok + 16 * t + r16], cn[1], O, 0, 0, 0);
#pragma unroll
            for (int v = 0; v < 4; ++v) blk[t][v] = O[v];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int g = j >> 1, sh = 4 * (j & 1);
            const int src = 4 * (r16 + 16 * (j >> 1));
            const float a = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, ca[j & 1])));
            const float cf = __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src, __builtin_bit_cast(int, cc[j & 1])));
            uint32_t c0 = (qq[2 * g] >> sh) & 0x0F0F0F0Fu, c1 = (qq[2 * g + 1] >> sh) & 0x0F0F0F0Fu;
            if constexpr (FMT == KQ_Q5_K) {
                c0 |= ((hh[0] >> j) & 0x01010101u) << 4;
                c1 |= ((hh[1] >> j) & 0x01010101u) << 4;
            }
            const uint2 p0 = codes_bf16(c0, cf), p1 = codes_bf16(c1, cf);
            const bf16x8_t bq = __builtin_bit_cast(bf16x8_t, make_uint4(p0.x, p0.y, p1.x, p1.y));
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const int off = (16 * t + r16) * kMbRow + 64 * j + 16 * h;
                const bf16x8_t xh = *reinterpret_cast<const bf16x8_t*>(xh_base + off);
                const bf16x8_t xl = *reinterpret_cast<const bf16x8_t*>(xl_base + off);
                f32x4 C = {0.0f, 0.0f, 0.0f, 0.0f};
                C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xh, bq, C, 0, 0, 0);
                C = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xl, bq, C, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) blk[t][v] = __builtin_fmaf(a, C[v], blk[t][v]);
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] += blk[t][v];
    }
    if constexpr (KS > 1) {
        // the tile's KS partial sums, added in wave order by its first wave
        static_assert(NW * TT * 4 * 64 * 4 <= KS * kPlane, "the partial sums fit in the x plane");
        float* part = reinterpret_cast<float*>(xs[0]);
        __syncthreads();                                    // every wave is done with x
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[((wave * TT + t) * 4 + v) * 64 + lane] = acc[t][v];
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int k = 1; k < KS; ++k) acc[t][v] += part[(((wave + k) * TT + t) * 4 + v) * 64 + lane];
    }
    const int row = row0 + r16;
    if (row < rows) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * t + 4 * h + v;
                if (tok < ntok) y[(int64_t)tok * ldy + row] = acc[t][v];
            }
    }
}

// Q6_K on the bf16 matrix cores: W = d*sc_j*(q - 32) over 16-element
// sub-blocks j, each with its own scale (muser-book Ch 6 Figure 6.5), so
// each sub-block takes 16x16x16 products: the codes q - 32 (six bits,
// exact in bf16) against x's two bf16 parts, C_j = sum (q - 32)*(hi + lo),
// then y += d * sum_j sc_j*C_j (no minimum term, every error relative to
// |W_e x_e|).  Lane l supplies row l % 16 (and token l % 16) over elements
// 16j + 4*(l/16) .. +3, whose codes are bytes of one ql word and one qh
// word of the row's block.
template <int TT, int KS, int NW>
__global__ __launch_bounds__(64 * NW) void kq_mmb6_kernel(const uint8_t* w, int64_t row_bytes, int32_t rows,
                                                          int32_t nb, const float* x, int64_t ldx, int32_t ntok,
                                                          float* y, int64_t ldy) {
    static_assert(KS == 1 || KS == 2 || KS == 4, "1, 2 or 4 waves a tile");
    static_assert(NW == 4 || NW == 8, "four or eight waves a workgroup");
    constexpr int BB = 210;
    constexpr int kTok = 16 * TT;
    constexpr int kXP = 16 * TT / NW;
    constexpr int kXR = kXP * KS;
    constexpr int kPlane = kTok * kMbRow;
    __shared__ __attribute__((aligned(16))) uint8_t xs[2][KS * kPlane];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, r16 = lane & 15, h = lane >> 4;
    const int ks = wave % KS;
    const int row0 = (blockIdx.x * (NW / KS) + wave / KS) * 16;
    const int tok0 = blockIdx.y * kTok;
    const int steps = (nb + KS - 1) / KS;
    const uint8_t* arow = w + (int64_t)min(row0 + r16, rows - 1) * row_bytes;
    const float* xcol = x + 4 * (tid & 63);
    const int xtok = tok0 + (tid >> 6);
    float acc[TT][4];
#pragma unroll
    for (int t = 0; t < TT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[t][v] = 0.0f;
    u32x4 xr[kXR];
    // the lane's words of the block, read as aligned words from the block's
    // 4-byte-aligned base a: ql bytes 64n + 32t + 16u + 4h .. +3 (words
    // 16n + 8t + 4u + h and the next), qh bytes 128 + 32n + 16u + 4h .. +3
    // (words 32 + 8n + 4u + h and the next), the scales (words 48..51, and
    // word 52 only when the block starts two bytes into a word), d (the two
    // bytes at 208).  The highest word read is 48 for ql/qh; word 52 lies
    // inside a block that starts two bytes into a word, so nothing past
    // byte 209 of the block is read.
    uint32_t wq[8][2], wh[4][2], wsc[5], wd, wsh;
    auto load = [&](int st) {
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            const int64_t xb = 256 * (int64_t)min(st * KS + k, nb - 1);
#pragma unroll
            for (int i = 0; i < kXP; ++i)
                xr[k * kXP + i] =
                    *reinterpret_cast<const u32x4*>(xcol + (int64_t)min(xtok + NW * i, ntok - 1) * ldx + xb);
        }
        const uint8_t* blk = arow + (int64_t)min(st * KS + ks, nb - 1) * BB;
        const uint32_t* a = reinterpret_cast<const uint32_t*>(reinterpret_cast<uintptr_t>(blk) & ~(uintptr_t)3);
        wsh = (reinterpret_cast<uintptr_t>(blk) & 2) ? 16u : 0u;
#pragma unroll
        for (int i = 0; i < 8; ++i) {                      // i = 4n + 2t + u
            wq[i][0] = a[16 * (i >> 2) + 8 * ((i >> 1) & 1) + 4 * (i & 1) + h];
            wq[i][1] = a[16 * (i >> 2) + 8 * ((i >> 1) & 1) + 4 * (i & 1) + h + 1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {                      // i = 2n + u
            wh[i][0] = a[32 + 8 * (i >> 1) + 4 * (i & 1) + h];
            wh[i][1] = a[32 + 8 * (i >> 1) + 4 * (i & 1) + h + 1];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) wsc[i] = a[48 + i];
        wsc[4] = a[51 + (wsh >> 4)];
        wd = *reinterpret_cast<const uint16_t*>(blk + 208);
    };
    load(0);
    for (int st = 0; st < steps; ++st) {
        __syncthreads();                                    // the previous step's LDS reads are done
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int i = 0; i < kXP; ++i) {
                uint2 hi, lo;
                split_x(__builtin_bit_cast(float4, xr[k * kXP + i]), hi, lo);
                const int off = k * kPlane + ((tid >> 6) + NW * i) * kMbRow + 8 * (tid & 63);
                *reinterpret_cast<uint2*>(xs[0] + off) = hi;
                *reinterpret_cast<uint2*>(xs[1] + off) = lo;
            }
        uint32_t ql[8], qh[4], sc[4];
#pragma unroll
        for (int i = 0; i < 8; ++i) ql[i] = __builtin_amdgcn_alignbit(wq[i][1], wq[i][0], wsh);
#pragma unroll
        for (int i = 0; i < 4; ++i) qh[i] = __builtin_amdgcn_alignbit(wh[i][1], wh[i][0], wsh);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[i] = __builtin_amdgcn_alignbit(wsc[i + 1], wsc[i], wsh);
        const float d = f16_to_f32(wd);
        __syncthreads();                                    // x of the step's blocks is in LDS
        load(min(st + 1, steps - 1));
        asm volatile("" : : : "memory");
        if (st * KS + ks >= nb) continue;                   // a ragged last step (the wave's own block)
        const uint8_t* xh_base = xs[0] + ks * kPlane;
        const uint8_t* xl_base = xs[1] + ks * kPlane;
        float blk[TT][4];
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) blk[t][v] = 0.0f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int n = j >> 3, s = (j >> 1) & 3, u = j & 1;
            const uint32_t lo4 = (ql[4 * n + 2 * (s & 1) + u] >> (4 * (s >> 1))) & 0x0F0F0F0Fu;
            const uint32_t hi2 = ((qh[2 * n + u] >> (2 * s)) & 0x03030303u) << 4;
            const uint2 p = codes_bf16(lo4 | hi2, 32.0f);
            const short4_t bq = __builtin_bit_cast(short4_t, p);
            const float scj = (float)((int32_t)(sc[j >> 2] << (24 - 8 * (j & 3))) >> 24);   // exact
#pragma unroll
            for (int t = 0; t < TT; ++t) {
                const int off = (16 * t + r16) * kMbRow + 32 * j + 8 * h;
                const short4_t xh = __builtin_bit_cast(short4_t, *reinterpret_cast<const uint2*>(xh_base + off));
                const short4_t xl = __builtin_bit_cast(short4_t, *reinterpret_cast<const uint2*>(xl_base + off));
                f32x4 C = {0.0f, 0.0f, 0.0f, 0.0f};
                C = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xh, bq, C, 0, 0, 0);
                C = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(xl, bq, C, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) blk[t][v] = __builtin_fmaf(scj, C[v], blk[t][v]);
            }
        }
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[t][v] = __builtin_fmaf(d, blk[t][v], acc[t][v]);
    }
    if constexpr (KS > 1) {
        static_assert(NW * TT * 4 * 64 * 4 <= KS * kPlane, "the partial sums fit in the x plane");
        float* part = reinterpret_cast<float*>(xs[0]);
        __syncthreads();
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) part[((wave * TT + t) * 4 + v) * 64 + lane] = acc[t][v];
        __syncthreads();
        if (ks != 0) return;
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int k = 1; k < KS; ++k) acc[t][v] += part[(((wave + k) * TT + t) * 4 + v) * 64 + lane];
    }
    const int row = row0 + r16;
    if (row < rows) {
#pragma unroll
        for (int t = 0; t < TT; ++t)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = tok0 + 16 * t + 4 * h + v;
                if (tok < ntok) y[(int64_t)tok * ldy + row] = acc[t][v];
            }
    }
}

int launch_matmul(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
                  int64_t ldy, int32_t ntok, hipStream_t stream) {
    const int32_t nb = (int32_t)(cols / 256);
    const int64_t row_bytes = (int64_t)nb * (fmt == KQ_Q4_K ? 144 : fmt == KQ_Q5_K ? 176 : 210);
    // 32 tokens a workgroup: two 16-token tiles (four tiles need more
    // accumulator and staging registers than fit two waves a SIMD, and ran
    // slower); Q4_K/Q5_K take eight row tiles a workgroup (four: the
    // attention output 197 -> 175 us), Q6_K four
    const dim3 grid((unsigned)((rows + 63) / 64), (unsigned)((ntok + 31) / 32));
    const dim3 grid8((unsigned)((rows + 127) / 128), grid.y);
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    switch (fmt) {
    case KQ_Q4_K:
        hipLaunchKernelGGL((kq_mmb_kernel<KQ_Q4_K, 2, 1, 8>), grid8, dim3(512), 0, stream, wb, row_bytes, (int32_t)rows,
                           nb, x, ldx, ntok, y, ldy);
        break;
    case KQ_Q5_K:
        hipLaunchKernelGGL((kq_mmb_kernel<KQ_Q5_K, 2, 1, 8>), grid8, dim3(512), 0, stream, wb, row_bytes, (int32_t)rows,
                           nb, x, ldx, ntok, y, ldy);
        break;
    default:
        hipLaunchKernelGGL((kq_mmb6_kernel<2, 1, 8>), grid8, dim3(512), 0, stream, wb, row_bytes, (int32_t)rows, nb,
                           x, ldx, ntok, y, ldy);
        break;
    }
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

int launch_matvec16(int32_t fmt, const void* w, int64_t rows, int64_t cols, const float* x, int64_t ldx, float* y,
                    int64_t ldy, int32_t ntok, hipStream_t stream) {
    const int32_t nb = (int32_t)(cols / 256);
    const int64_t row_bytes = (int64_t)nb * (fmt == KQ_Q4_K ? 144 : fmt == KQ_Q5_K ? 176 : 210);
    const int64_t tiles = (rows + 15) / 16;
    const uint8_t* wb = static_cast<const uint8_t*>(w);
    // bf16 matrix products, eight waves a workgroup (four: the attention
    // output 17.1 -> 20.4 us); a tile's blocks split over 4 / 2 waves while
    // there are at most 512 / 2048 tiles (the row count alone decides; 4
    // waves up to 2048 tiles: the FFN gate 59 -> 78 us)
    const int ks = tiles <= 512 ? 4 : tiles <= 2048 ? 2 : 1;
    const dim3 g((unsigned)((tiles * ks + 7) / 8));
#define KQ_MMB16(KERNEL)                                                                                         \
    hipLaunchKernelGGL(KERNEL, g, dim3(512), 0, stream, wb, row_bytes, (int32_t)rows, nb, x, ldx, ntok, y, ldy)
    if (fmt == KQ_Q4_K) {
        if (ks == 4) KQ_MMB16((kq_mmb_kernel<KQ_Q4_K, 1, 4, 8>));
        else if (ks == 2) KQ_MMB16((kq_mmb_kernel<KQ_Q4_K, 1, 2, 8>));
        else KQ_MMB16((kq_mmb_kernel<KQ_Q4_K, 1, 1, 8>));
    } else if (fmt == KQ_Q5_K) {
        if (ks == 4) KQ_MMB16((kq_mmb_kernel<KQ_Q5_K, 1, 4, 8>));
        else if (ks == 2) KQ_MMB16((kq_mmb_kernel<KQ_Q5_K, 1, 2, 8>));
        else KQ_MMB16((kq_mmb_kernel<KQ_Q5_K, 1, 1, 8>));
    } else {
        if (ks == 4) KQ_MMB16((kq_mmb6_kernel<1, 4, 8>));
        else if (ks == 2) KQ_MMB16((kq_mmb6_kernel<1, 2, 8>));
        else KQ_MMB16((kq_mmb6_kernel<1, 1, 8>));
    }
#undef KQ_MMB16
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

// ------------------------------------------------------------ debug kernels
// One thread per super-block: fetch the block's aligned words, decode with
// the same helpers as the matvec, expand to integers / float weights.
__device__ void load_block_words(int32_t fmt, const uint8_t* w, int64_t blk, uint32_t* E) {
    const int bb = (fmt == KQ_Q4_K) ? 144 : (fmt == KQ_Q5_K) ? 176 : 210;
    const uint8_t* p = w + blk * bb;
    const size_t mis = reinterpret_cast<uintptr_t>(p) & 3;     // 0 or 2 (Q6_K odd blocks)
    const uint32_t* a = reinterpret_cast<const uint32_t*>(p - mis);
    const int words = (bb + 3) / 4;   // 53 words cover [p-2, p+210) when mis == 2
    for (int i = 0; i < words; ++i) E[i] = a[i];
    if (mis) {
        E[words] = 0;
        for (int i = 0; i < words; ++i) E[i] = align2(E[i], E[i + 1]);
    }
}

__global__ void kq_unpack_kernel(int32_t fmt, const uint8_t* w, int64_t nblocks, int32_t* codes,
                                 int32_t* scales, int32_t* mins, float* dv, float* dminv) {
    const int64_t blk = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (blk >= nblocks) return;
    uint32_t E[56];
    for (int i = 0; i < 56; ++i) E[i] = 0;
    // Q6_K even blocks: the final word holds bytes 208..211; read it as 2 bytes
    if (fmt == KQ_Q6_K && (blk & 1) == 0) {
        const uint8_t* p = w + blk * 210;
        const uint32_t* a = reinterpret_cast<const uint32_t*>(p);
        for (int i = 0; i < 52; ++i) E[i] = a[i];
        E[52] = *reinterpret_cast<const uint16_t*>(p + 208);
    } else {
        load_block_words(fmt, w, blk, E);
    }
    int32_t* cq = codes ? codes + blk * 256 : nullptr;
    if (fmt == KQ_Q4_K || fmt == KQ_Q5_K) {
        const K4Scales S = k4_scales(E[1], E[2], E[3]);
        if (scales) for (int j = 0; j < 16; ++j) scales[blk * 16 + j] = j < 8 ? (int32_t)k4_sc(S, j) : 0;
        if (mins) for (int j = 0; j < 16; ++j) mins[blk * 16 + j] = j < 8 ? (int32_t)k4_m(S, j) : 0;
        if (dv) dv[blk] = f16_to_f32(E[0] & 0xFFFFu);
        if (dminv) dminv[blk] = f16_to_f32(E[0] >> 16);
        if (cq) {
            const int qs = (fmt == KQ_Q4_K) ? 4 : 12;
            for (int g = 0; g < 4; ++g) {
                for (int k = 0; k < 8; ++k) {
                    Packed4 p;
                    const uint32_t q = E[qs + 8 * g + k];
                    if (fmt == KQ_Q4_K) p = k4_codes(q);
                    else if (g == 0) p = k5_codes<0>(q, E[4 + k]);
                    else if (g == 1) p = k5_codes<1>(q, E[4 + k]);
                    else if (g == 2) p = k5_codes<2>(q, E[4 + k]);
                    else p = k5_codes<3>(q, E[4 + k]);
                    const int e = 64 * g + 4 * k;
                    cq[e + 0] = p.lo02 & 0xFFFF;  cq[e + 2] = p.lo02 >> 16;
                    cq[e + 1] = p.lo13 & 0xFFFF;  cq[e + 3] = p.lo13 >> 16;
                    cq[e + 32] = (p.hi02 & 0xFFFF) >> 4;  cq[e + 34] = (p.hi02 >> 16) >> 4;
                    cq[e + 33] = (p.hi13 & 0xFFFF) >> 4;  cq[e + 35] = (p.hi13 >> 16) >> 4;
                }
            }
        }
    } else {
        if (scales) for (int j = 0; j < 16; ++j) scales[blk * 16 + j] = (int8_t)(E[48 + j / 4] >> (8 * (j % 4)));
        if (mins) for (int j = 0; j < 16; ++j) mins[blk * 16 + j] = 0;
        if (dv) dv[blk] = f16_to_f32(E[52] & 0xFFFFu);
        if (dminv) dminv[blk] = 0.0f;
        if (cq) {
            for (int n = 0; n < 2; ++n) {
                for (int k = 0; k < 8; ++k) {
                    const Packed6 p = k6_codes(E[16 * n + k], E[16 * n + 8 + k], E[32 + 8 * n + k]);
                    for (int c = 0; c < 4; ++c) {
                        const int e = 128 * n + 32 * c + 4 * k;
                        const int sh = c < 2 ? 0 : 4;
                        cq[e + 0] = (int32_t)((p.c02[c] & 0xFFFF) >> sh) - 32;
                        cq[e + 2] = (int32_t)((p.c02[c] >> 16) >> sh) - 32;
                        cq[e + 1] = (int32_t)((p.c13[c] & 0xFFFF) >> sh) - 32;
                        cq[e + 3] = (int32_t)((p.c13[c] >> 16) >> sh) - 32;
                    }
                }
            }
        }
    }
}

__global__ void kq_dequant_kernel(int32_t fmt, const uint8_t* w, int64_t rows, int32_t nb, float* out,
                                  int64_t ldw) {
    const int64_t blk = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
    if (blk >= rows * nb) return;
    const int64_t r = blk / nb, b = blk - (blk / nb) * nb;
    int32_t codes[256], sc[16], mn[16];
    float d, dmin;
    // reuse the unpack path's decode, one block, in registers/scratch
    uint32_t E[56];
    for (int i = 0; i < 56; ++i) E[i] = 0;
    if (fmt == KQ_Q6_K && (blk & 1) == 0) {
        const uint8_t* p = w + blk * 210;
        const uint32_t* a = reinterpret_cast<const uint32_t*>(p);
        for (int i = 0; i < 52; ++i) E[i] = a[i];
        E[52] = *reinterpret_cast<const uint16_t*>(p + 208);
    } else {
        load_block_words(fmt, w, blk, E);
    }
    float* o = out + r * ldw + 256 * b;
    if (fmt == KQ_Q4_K || fmt == KQ_Q5_K) {
        const K4Scales S = k4_scales(E[1], E[2], E[3]);
        d = f16_to_f32(E[0] & 0xFFFFu);
        dmin = f16_to_f32(E[0] >> 16);
        const int qs = (fmt == KQ_Q4_K) ? 4 : 12;
        for (int g = 0; g < 4; ++g) {
            for (int k = 0; k < 8; ++k) {
                Packed4 p;
                const uint32_t q = E[qs + 8 * g + k];
                if (fmt == KQ_Q4_K) p = k4_codes(q);
                else if (g == 0) p = k5_codes<0>(q, E[4 + k]);
                else if (g == 1) p = k5_codes<1>(q, E[4 + k]);
                else if (g == 2) p = k5_codes<2>(q, E[4 + k]);
                else p = k5_codes<3>(q, E[4 + k]);
                const int e = 64 * g + 4 * k;
                codes[e + 0] = p.lo02 & 0xFFFF;  codes[e + 2] = p.lo02 >> 16;
                codes[e + 1] = p.lo13 & 0xFFFF;  codes[e + 3] = p.lo13 >> 16;
                codes[e + 32] = (p.hi02 & 0xFFFF) >> 4;  codes[e + 34] = (p.hi02 >> 16) >> 4;
                codes[e + 33] = (p.hi13 & 0xFFFF) >> 4;  codes[e + 35] = (p.hi13 >> 16) >> 4;
            }
        }
        for (int j = 0; j < 8; ++j) { sc[j] = k4_sc(S, j); mn[j] = k4_m(S, j); }
        for (int e = 0; e < 256; ++e) {
            const int j = e / 32;
            const float a = (d * (float)sc[j]) * (float)codes[e];   // exact
            const float m = dmin * (float)mn[j];                     // exact
            o[e] = a - m;                                            // one rounding
        }
    } else {
        d = f16_to_f32(E[52] & 0xFFFFu);
        for (int j = 0; j < 16; ++j) sc[j] = (int8_t)(E[48 + j / 4] >> (8 * (j % 4)));
        for (int n = 0; n < 2; ++n) {
            for (int k = 0; k < 8; ++k) {
                const Packed6 p = k6_codes(E[16 * n + k], E[16 * n + 8 + k], E[32 + 8 * n + k]);
                for (int c = 0; c < 4; ++c) {
                    const int e = 128 * n + 32 * c + 4 * k;
                    const int sh = c < 2 ? 0 : 4;
                    codes[e + 0] = (int32_t)((p.c02[c] & 0xFFFF) >> sh) - 32;
                    codes[e + 2] = (int32_t)((p.c02[c] >> 16) >> sh) - 32;
                    codes[e + 1] = (int32_t)((p.c13[c] & 0xFFFF) >> sh) - 32;
                    codes[e + 3] = (int32_t)((p.c13[c] >> 16) >> sh) - 32;
                }
            }
        }
        for (int e = 0; e < 256; ++e) o[e] = (d * (float)sc[e / 16]) * (float)codes[e];   // exact
    }
    (void)dmin;
}

// ------------------------------------------------------------ read probe
// A trivial streaming read (16-byte nontemporal loads, eight in flight per
// thread, XOR reduction): what HBM delivers to a kernel that does nothing
// else, the calibration the matvec's bandwidth is read against.  Writes
// *sink only if the XOR hits a fixed value, so the loads cannot be dropped.
__global__ __launch_bounds__(256) void kq_read_probe_kernel(const u32x4* __restrict__ p, int64_t n,
                                                             uint32_t* sink) {
    constexpr int U = 8;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) acc ^= p[i].x;
    if (acc == 0x9E3779B9u) sink[0] = acc;
}

int launch_read_probe(const void* buf, int64_t bytes, uint32_t* sink, hipStream_t stream) {
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return KQ_ERR_HIP;
    hipLaunchKernelGGL(kq_read_probe_kernel, dim3(cus * 32), dim3(256), 0, stream,
                       static_cast<const u32x4*>(buf), bytes / 16, sink);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

// ------------------------------------------------------------ launchers
// At most two waves per SIMD: more resident waves (the kernel would fit
// three at one token plane) spread the same bytes over more concurrent row
// streams and measured slower on large matrices.
#ifndef KQ_MAX_WAVES_PER_CU
#define KQ_MAX_WAVES_PER_CU 8
#endif
constexpr int kMaxWavesPerCU = KQ_MAX_WAVES_PER_CU;

// Resident one-wave workgroups per compute unit for this kernel and LDS
// size (queried once per device, token count and LDS size).
template <int NTOK>
static int resident_per_cu(int lds_bytes) {
    int dev = 0, per_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static int cache[16][9][4] = {};     // [device][ntok][lds class]
    const int cls = lds_bytes <= 12 * 1024 ? 0 : lds_bytes <= 20 * 1024 ? 1 : lds_bytes <= 28 * 1024 ? 2 : 3;
    int& c = cache[dev & 15][NTOK][cls];
    if (c == 0) {
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kq_matvec_kernel<NTOK>, 64, lds_bytes) != hipSuccess ||
            per_cu <= 0)
            per_cu = 1;
        c = per_cu;
    }
    return c;
}

static int compute_units() {
    static int cus[16] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int& c = cus[dev & 15];
    if (c == 0 && hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) c = 0;
    return c;
}

template <int NTOK>
static int capacity_t(int lds_bytes) {
    const int cus = compute_units();
    if (cus <= 0) return KQ_ERR_HIP;
    return min(resident_per_cu<NTOK>(lds_bytes), kMaxWavesPerCU) * cus;
}

// Whether launches may take the pipelined kernel: 1 (the default) when
// they are large enough, 0 never (the environment's KQMV_PIPELINE=0, or
// kq_debug_set_pipeline), 2 whenever they fit (kq_debug_set_pipeline: tests
// of small shapes).
static int g_pipeline = -1;
void set_pipeline(int mode) { g_pipeline = mode < 0 ? 0 : mode > 2 ? 2 : mode; }
static int pipeline_mode() {
    if (g_pipeline < 0) {
        const char* e = getenv("KQMV_PIPELINE");
        g_pipeline = (e && e[0] == '0') ? 0 : 1;
    }
    return g_pipeline;
}

// A launch of fewer steps than this many a compute unit takes the one-wave
// kernel: with a step or two a workgroup the pipeline never fills, and the
// one-wave kernel's smaller workgroups start sooner (a 256 x 6656 Q4_K
// matrix 7.6 -> 7.1 us, the 256-row Q6_K + Q5_K pair 9.1 -> 8.7 us; at
// 6.5 steps a compute unit the two kernels are level).
constexpr int kPcMinStepsPerCU = 4;

// A launch of at most this many steps a compute unit loads its weights with
// the non-temporal hint.  Measured back to back on one box, against the
// same kernel with ordinary loads: a decode set (14 steps a compute unit)
// 14.73 -> 14.43 us, 16 rotating sets 13.92 -> 13.38 us, the attention
// output (6.5 steps) 10.75 -> 10.56 us, the FFN gate + up (63 steps) 37.8
// -> 37.4 us; the 202,048-row matrices (320 steps) no faster, and their HBM
// traffic rose from 1.021 to 1.053 times their bytes.
constexpr int kPcNtMaxStepsPerCU = 128;

// Sets L up for the pipelined kernel when every tensor runs in 32-row tiles
// at ntok <= 2, the launch has enough steps (kPcMinStepsPerCU) and each
// tensor's resident x, its fold slots and a ring of at least kPcMinSlots
// steps fit one workgroup's LDS: each
// descriptor gets its ring slots R (even, at most 16) and fold slots TS, the
// launch its LDS size.  Returns
// whether it did (L->pipelined).
int plan_pipelined(KqLaunch* L) {
    L->pipelined = 0;
    const int mode = pipeline_mode();
    if (mode == 0 || L->ntok > 2) return 0;
    static int lds_max[16] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    int& lm = lds_max[dev & 15];
    if (lm == 0 && (hipDeviceGetAttribute(&lm, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lm <= 0))
        lm = -1;
    if (lm < 0) return 0;
    const int budget = lm - (int)sizeof(uint32_t) * PcLayout::words - 64;
    int lds = 0;
    for (int i = 0; i < L->h.n; ++i) {
        if (L->t[i].tile_rows != 32) return 0;
    }
    if (mode == 1 && L->total_segments < kPcMinStepsPerCU * compute_units()) return 0;
    const int nt = L->total_segments <= kPcNtMaxStepsPerCU * compute_units() ? 1 : 0;
    for (int i = 0; i < L->h.n; ++i) {
        KqDesc& D = L->t[i];
        int wb = 0, xb = 0, d = 0;
        pc_sizes(D.fmt, L->ntok, &wb, &xb, &d);
        // fold slots: the tiles the consumers' positions can span, plus two
        const int TS = min(kPcMaxFold, 2 + (kPcConsumers + D.nseg - 1) / D.nseg);
        const int sums = TS * D.nseg * L->ntok * 128, x_bytes = D.nseg * xb;
        // weight slots: what the rest of the LDS holds (even, at most
        // kPcMaxSlots), at least kPcMinSlots (and every producer's steps in
        // flight), or the launch takes kq_matvec_kernel
        int R = (budget - sums - x_bytes) / wb;
        R = (R > kPcMaxSlots ? kPcMaxSlots : R) & ~1;
        if (R < kPcMinSlots || R < kPcProducers * d) return 0;
        D.reserved0 = R | (TS << 8) | (nt << 16);
        const int need = R * wb + x_bytes + sums;
        if (need > lds) lds = need;
    }
    L->lds_bytes = lds;
    L->pipelined = 1;
    return 1;
}

// One round of resident workgroups for L on the current device: one
// workgroup a compute unit for the pipelined kernel, else one-wave
// workgroups of kq_matvec_kernel<ntok> with L's LDS size (at most two waves
// a SIMD).
int launch_capacity(const KqLaunch& L) {
    if (L.pipelined) return compute_units();
    const int32_t lds_bytes = L.lds_bytes;
    switch (L.ntok) {
    case 1: return capacity_t<1>(lds_bytes);
    case 2: return capacity_t<2>(lds_bytes);
    case 3: return capacity_t<3>(lds_bytes);
    case 4: return capacity_t<4>(lds_bytes);
    case 5: return capacity_t<5>(lds_bytes);
    case 6: return capacity_t<6>(lds_bytes);
    case 7: return capacity_t<7>(lds_bytes);
    default: return capacity_t<8>(lds_bytes);
    }
}

// The launch L, fully planned (workgroups assigned, workspace set).
int launch_matvec(const KqLaunch& L, hipStream_t stream) {
    const dim3 grid((unsigned)L.grid), block(64);
    const size_t lds = (size_t)L.lds_bytes;
    if (L.pipelined) {
        if (L.ntok == 1) hipLaunchKernelGGL(kq_pc_kernel<1>, grid, dim3(64 * kPcWaves), lds, stream, L);
        else hipLaunchKernelGGL(kq_pc_kernel<2>, grid, dim3(64 * kPcWaves), lds, stream, L);
        return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
    }
    switch (L.ntok) {
    case 1: hipLaunchKernelGGL(kq_matvec_kernel<1>, grid, block, lds, stream, L); break;
    case 2: hipLaunchKernelGGL(kq_matvec_kernel<2>, grid, block, lds, stream, L); break;
    case 3: hipLaunchKernelGGL(kq_matvec_kernel<3>, grid, block, lds, stream, L); break;
    case 4: hipLaunchKernelGGL(kq_matvec_kernel<4>, grid, block, lds, stream, L); break;
    case 5: hipLaunchKernelGGL(kq_matvec_kernel<5>, grid, block, lds, stream, L); break;
    case 6: hipLaunchKernelGGL(kq_matvec_kernel<6>, grid, block, lds, stream, L); break;
    case 7: hipLaunchKernelGGL(kq_matvec_kernel<7>, grid, block, lds, stream, L); break;
    default: hipLaunchKernelGGL(kq_matvec_kernel<8>, grid, block, lds, stream, L); break;
    }
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

// Zeroes n words at p on `stream` (a fill kernel, not a memset node, so
// the call can sit in a captured graph).
__global__ void kq_zero_kernel(uint32_t* p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

int launch_zero(uint32_t* p, int64_t n, hipStream_t stream) {
    if (n <= 0) return KQ_OK;
    hipLaunchKernelGGL(kq_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, n);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

// ------------------------------------------------------------ scratch of the allocation-free set call
// kq_matvec_set_noalloc takes its shared-tile sums and arrival counters from
// this array instead of a workspace it allocates.  Every call on a GPU uses
// that GPU's copy of the array, so calls that overlap on one GPU race.  In
// host code the array's name is a stand-in, not a device address: set-up
// takes each device's address once with hipGetSymbolAddress (with that
// device current), and only that address reaches kernels.
constexpr size_t kScratchFloats = (size_t)4 << 20;         // 16 MB of shared-tile sums
constexpr size_t kScratchCounters = (size_t)1 << 16;       // 65,536 arrival counters
constexpr size_t kScratchBytes = kScratchFloats * sizeof(float) + kScratchCounters * sizeof(uint32_t);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

static std::mutex g_scratch_mutex;
static void* g_scratch_addr[16];                            // per device, set once

// The scratch's sums and counters on the current device for a plan that
// needs `floats` sums and `counters` counters; KQ_ERR_SCRATCH when that is
// more than the array holds.  The first call on a device takes the array's
// address and zeroes its counters with a fill kernel on `stream` (every
// launch leaves the counters it used at zero again).  Allocates nothing.
int scratch_workspace(hipStream_t stream, size_t floats, size_t counters, float** partials, uint32_t** ctrs) {
    *partials = nullptr;
    *ctrs = nullptr;
    if (floats > kScratchFloats || counters > kScratchCounters) return KQ_ERR_SCRATCH;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return KQ_ERR_HIP;
    void* base = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_scratch_mutex);
        if (g_scratch_addr[dev] == nullptr) {
            void* p = nullptr;
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return KQ_ERR_HIP;
            uint32_t* c = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(p) + kScratchFloats * sizeof(float));
            if (launch_zero(c, (int64_t)kScratchCounters, stream) != KQ_OK) return KQ_ERR_HIP;
            g_scratch_addr[dev] = p;
        }
        base = g_scratch_addr[dev];
    }
    *partials = static_cast<float*>(base);
    *ctrs = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + kScratchFloats * sizeof(float));
    return KQ_OK;
}

int launch_unpack(int32_t fmt, const void* w, int64_t nblocks, int32_t* codes, int32_t* scales,
                  int32_t* mins, float* d, float* dmin, hipStream_t stream) {
    const int64_t grid = (nblocks + 255) / 256;
    hipLaunchKernelGGL(kq_unpack_kernel, dim3((unsigned)grid), dim3(256), 0, stream, fmt,
                       static_cast<const uint8_t*>(w), nblocks, codes, scales, mins, d, dmin);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

int launch_dequant(int32_t fmt, const void* w, int64_t rows, int32_t nb, float* out, int64_t ldw,
                   hipStream_t stream) {
    const int64_t grid = (rows * nb + 255) / 256;
    hipLaunchKernelGGL(kq_dequant_kernel, dim3((unsigned)grid), dim3(256), 0, stream, fmt,
                       static_cast<const uint8_t*>(w), rows, nb, out, ldw);
    return hipGetLastError() == hipSuccess ? KQ_OK : KQ_ERR_HIP;
}

}  // namespace kq
