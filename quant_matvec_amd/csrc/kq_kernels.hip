// kq_kernels.hip -- gfx950 kernels of the k-quant decode matvec.
//
// y = W x with W in k-quant super-blocks, dequantized in registers and
// never stored (muser-book Ch 13 "The QKV + gate matvec family", section
// 13.1; formats from muser-book Ch 6 sections 6.2-6.4).
//
// Mapping (one wave64 per workgroup, see kq_plan.h for the items):
//   * lane i owns output row r0+i, so all 64 lanes walk the same super-block
//     column at the same time.  The x values a multiply-add needs are then
//     the same for the whole wave: they are read with scalar loads into
//     SGPRs and used directly as an operand of v_fma_mix_f32, costing no
//     VGPRs, no LDS bandwidth and no per-lane memory traffic.
//   * The 64 rows of a super-block column are strided in HBM (one row every
//     row_bytes).  They are fetched with coalesced 16-byte loads (4-byte
//     loads for the 210-byte Q6_K blocks) into registers, written to a
//     per-wave LDS slot, and read back one row per lane: a transpose through
//     LDS.  The next column's loads are issued before the current column is
//     computed, so one column is always in flight per wave.
//   * Codes become binary16 subnormals two per word (kq_decode.h) and feed
//     v_fma_mix_f32 directly: one instruction per weight for the
//     multiply-add, plus about 0.6 (Q4_K) to 1.4 (Q6_K) bit operations per
//     weight to unpack.
//   * Scales are applied once per sub-block (deferred scaling, muser-book
//     Ch 13 section 13.4.2): per sub-block j the lane accumulates
//     sum(q*x) and adds d*sc_j*that - dmin*m_j*sum(x); sum(x) over each
//     sub-block is computed once per column by the wave with DPP reductions.
//   * No MFMA: at ntok <= 8 this is a streaming dot product, not a dense
//     contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kq_decode.h"
#include "kq_plan.h"

namespace kq {

typedef const float __attribute__((address_space(4)))* xconst_t;   // scalar-loadable view of x
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kTwo24 = 16777216.0f;        // undoes the 2^-24 of a subnormal code

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

// Sums of x over the sub-blocks of one super-block column, for one token
// plane xp: SUB = 32 (Q4_K/Q5_K, 8 sums) or 16 (Q6_K, 16 sums).  Lane i adds
// x[4i..4i+3]; groups of 8 (or 4) lanes are reduced with DPP, so afterwards
// every lane of group j holds the sum of sub-block j.  The order is fixed,
// so every workgroup gets the same bits.  The result stays in one VGPR and
// a sum is moved to an SGPR (readlane) only where it is used.
template <int SUB>
__device__ __forceinline__ float subblock_sums(const float* xp) {
    const int lane = threadIdx.x;
    float4 v = *reinterpret_cast<const float4*>(xp + 4 * lane);
    float s = (v.x + v.y) + (v.z + v.w);
    s = s + dpp_xor1(s);
    s = s + dpp_xor2(s);
    if (SUB == 32) s = s + dpp_half_mirror(s);
    return s;
}

// Workgroup id -> item.  Workgroups are dealt to the 8 XCDs round-robin;
// this gives each XCD a contiguous run of items, so the column-split items
// of one row tile (which share the cache lines at their boundaries) run on
// the same XCD and meet in its L2.
__device__ __forceinline__ int xcd_item(int bid, int nblocks) {
    const int xcd = bid & 7, local = bid >> 3;
    const int base = nblocks >> 3, rem = nblocks & 7;
    return xcd * base + min(xcd, rem) + local;
}

// ------------------------------------------------------------ item context
struct Item {
    int tile, kp, r0, rows_here, kb0, kb1;
};

__device__ __forceinline__ Item make_item(const KqDesc& T, int local) {
    Item it;
    it.tile = local / T.kparts;
    it.kp = local - it.tile * T.kparts;
    it.r0 = it.tile * kTileRows;
    it.rows_here = min(kTileRows, T.rows - it.r0);
    it.kb0 = it.kp * T.kchunk;
    it.kb1 = min(T.nb, it.kb0 + T.kchunk);
    return it;
}

// Write the 64 row results, or hand them to the column-split fix-up: the
// last item of a row tile to arrive adds all partials in column order.
template <int NTOK>
__device__ __forceinline__ void finish_item(const KqDesc& T, const KqLaunch& L, const Item& it,
                                            const float (&acc)[NTOK]) {
    const int lane = threadIdx.x;
    if (T.kparts == 1) {
        if (lane < it.rows_here) {
#pragma unroll
            for (int t = 0; t < NTOK; ++t) T.y[t * T.ldy + it.r0 + lane] = acc[t];
        }
        return;
    }
    float* tile_parts = L.partials + (size_t)(T.part_base + it.tile * T.kparts) * (NTOK * kTileRows);
    float* mine = tile_parts + (size_t)it.kp * (NTOK * kTileRows);
#pragma unroll
    for (int t = 0; t < NTOK; ++t)
        __hip_atomic_store(mine + t * kTileRows + lane, acc[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint32_t* ctr = L.counters + T.tile_base + it.tile;
    uint32_t old = 0;
    if (lane == 0) old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);
    if (old != (uint32_t)(T.kparts - 1)) return;
    // last arriver: every other item's partials are visible (acq_rel above)
    float sum[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) sum[t] = 0.0f;
    for (int p = 0; p < T.kparts; ++p) {
        const float* src = tile_parts + (size_t)p * (NTOK * kTileRows);
#pragma unroll
        for (int t = 0; t < NTOK; ++t)
            sum[t] += __hip_atomic_load(src + t * kTileRows + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (lane < it.rows_here) {
#pragma unroll
        for (int t = 0; t < NTOK; ++t) T.y[t * T.ldy + it.r0 + lane] = sum[t];
    }
    if (lane == 0) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint4 lds_read4(const uint8_t* p) { return *reinterpret_cast<const uint4*>(p); }
__device__ __forceinline__ uint32_t lds_read1(const uint8_t* p) { return *reinterpret_cast<const uint32_t*>(p); }

// ------------------------------------------------------------ Q4_K / Q5_K
// Block of 144 (Q4_K) or 176 (Q5_K) bytes = 9 or 11 16-byte chunks.
// Q4_K: d|dmin, strip[12], qs[128].  Q5_K: d|dmin, strip[12], qh[32], qs[128].
template <int FMT>
struct K45 {
    static constexpr int BB = (FMT == KQ_Q4_K) ? 144 : 176;
    static constexpr int C = BB / 16;                          // chunks per row = uint4 staged per lane
    static constexpr int QS_OFF = (FMT == KQ_Q4_K) ? 16 : 48;  // byte offset of qs
};

// One group g of a block: sub-blocks 2g (low nibbles) and 2g+1 (high).
template <int FMT, int NTOK, int G>
__device__ __forceinline__ void k45_group(const uint8_t* row, const uint32_t (&qh)[8], const K4Scales& S,
                                          xconst_t xb, int64_t ldx, const float (&sx)[NTOK],
                                          float (&ts_e)[NTOK], float (&ts_o)[NTOK], float (&tm)[NTOK]) {
    uint32_t qs[8];
    {
        const uint4 a = lds_read4(row + K45<FMT>::QS_OFF + 32 * G);
        const uint4 b = lds_read4(row + K45<FMT>::QS_OFF + 32 * G + 16);
        qs[0] = a.x; qs[1] = a.y; qs[2] = a.z; qs[3] = a.w;
        qs[4] = b.x; qs[5] = b.y; qs[6] = b.z; qs[7] = b.w;
    }
    float al[NTOK], ah[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) { al[t] = 0.0f; ah[t] = 0.0f; }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        Packed4 p;
        if constexpr (FMT == KQ_Q4_K) p = k4_codes(qs[k]);
        else p = k5_codes<G>(qs[k], qh[k]);
        const int e = 64 * G + 4 * k;
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            xconst_t xt = xb + t * ldx;
            al[t] = __builtin_fmaf((float)half_lo(p.lo02), xt[e + 0], al[t]);
            al[t] = __builtin_fmaf((float)half_lo(p.lo13), xt[e + 1], al[t]);
            al[t] = __builtin_fmaf((float)half_hi(p.lo02), xt[e + 2], al[t]);
            al[t] = __builtin_fmaf((float)half_hi(p.lo13), xt[e + 3], al[t]);
            ah[t] = __builtin_fmaf((float)half_lo(p.hi02), xt[e + 32], ah[t]);
            ah[t] = __builtin_fmaf((float)half_lo(p.hi13), xt[e + 33], ah[t]);
            ah[t] = __builtin_fmaf((float)half_hi(p.hi02), xt[e + 34], ah[t]);
            ah[t] = __builtin_fmaf((float)half_hi(p.hi13), xt[e + 35], ah[t]);
        }
    }
    const float sc0 = (float)k4_sc(S, 2 * G), sc1 = (float)k4_sc(S, 2 * G + 1);
    const float m0 = (float)k4_m(S, 2 * G), m1 = (float)k4_m(S, 2 * G + 1);
#pragma unroll
    for (int t = 0; t < NTOK; ++t) {
        ts_e[t] = __builtin_fmaf(sc0, al[t], ts_e[t]);
        ts_o[t] = __builtin_fmaf(sc1, ah[t], ts_o[t]);
        tm[t] = __builtin_fmaf(m0, lane_value(sx[t], 8 * (2 * G)), tm[t]);
        tm[t] = __builtin_fmaf(m1, lane_value(sx[t], 8 * (2 * G + 1)), tm[t]);
    }
}

template <int FMT, int NTOK>
__device__ __forceinline__ void item_k45(const KqDesc& T, const KqLaunch& L, const Item& it, uint8_t* slot) {
    constexpr int C = K45<FMT>::C;
    constexpr int BB = K45<FMT>::BB;
    const int lane = threadIdx.x;
    const uint8_t* base = T.w + (size_t)it.r0 * T.row_bytes;

    // staging: 16-byte chunk q = 64*i + lane of the column -> row q / C, chunk q % C;
    // in LDS it lands at byte 16*q = row*BB + 16*chunk.
    uint4 stg[C];
    uint32_t off[C];
    const int nlive = it.rows_here * C;     // chunks that belong to existing rows
#pragma unroll
    for (int i = 0; i < C; ++i) {
        const int q = 64 * i + lane;
        const int r = q / C, c = q - (q / C) * C;
        off[i] = (uint32_t)r * (uint32_t)T.row_bytes + 16u * c;
        stg[i] = make_uint4(0, 0, 0, 0);
    }
    auto stage = [&](int b) {
        const uint8_t* col = base + (size_t)b * BB;
#pragma unroll
        for (int i = 0; i < C; ++i)
            if (64 * i + lane < nlive)
                stg[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(col + off[i])));
    };

    float acc[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = 0.0f;
    const uint8_t* row = slot + lane * BB;

    stage(it.kb0);
    for (int b = it.kb0; b < it.kb1; ++b) {
        __syncthreads();                            // earlier reads of the slot are done
#pragma unroll
        for (int i = 0; i < C; ++i) reinterpret_cast<uint4*>(slot)[64 * i + lane] = stg[i];
        if (b + 1 < it.kb1) stage(b + 1);           // next column in flight during this one

        float sx[NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) sx[t] = subblock_sums<32>(T.x + t * T.ldx + 256 * b);

        __syncthreads();                            // slot written
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
        const float d = f16_to_f32(hdr.x & 0xFFFFu), dmin = f16_to_f32(hdr.x >> 16);
        const K4Scales S = k4_scales(hdr.y, hdr.z, hdr.w);
        xconst_t xb = (xconst_t)(T.x) + 256 * b;
        float ts_e[NTOK], ts_o[NTOK], tm[NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) { ts_e[t] = 0.0f; ts_o[t] = 0.0f; tm[t] = 0.0f; }
        k45_group<FMT, NTOK, 0>(row, qh, S, xb, T.ldx, sx, ts_e, ts_o, tm);
        __builtin_amdgcn_sched_barrier(0);
        k45_group<FMT, NTOK, 1>(row, qh, S, xb, T.ldx, sx, ts_e, ts_o, tm);
        __builtin_amdgcn_sched_barrier(0);
        k45_group<FMT, NTOK, 2>(row, qh, S, xb, T.ldx, sx, ts_e, ts_o, tm);
        __builtin_amdgcn_sched_barrier(0);
        k45_group<FMT, NTOK, 3>(row, qh, S, xb, T.ldx, sx, ts_e, ts_o, tm);
        const float d24 = d * kTwo24;
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            const float v = __builtin_fmaf(ts_o[t], 0.0625f, ts_e[t]);   // odd sub-blocks were 16*code
            acc[t] = __builtin_fmaf(d24, v, acc[t]);
            acc[t] = __builtin_fmaf(-dmin, tm[t], acc[t]);
        }
    }
    finish_item<NTOK>(T, L, it, acc);
}

// -------------------------------------------------------------------- Q6_K
// 210-byte block: ql[128], qh[64], sc[16] (int8), d (f16, last).  A block
// starts 2 bytes into a word when its index in the tensor is odd, so each
// row's block is staged as the 53 aligned words covering it (one row per
// load instruction, lanes 0..52, all addressing uniform) into a 240-byte
// LDS row, and shifted by two bytes after the LDS read where needed.
constexpr int kQ6Words = 53;
constexpr int kQ6LdsRow = 240;

// The block's words w[i..i+3] (and w[i+4] for the shift) realigned.
__device__ __forceinline__ void q6_read4(const uint8_t* row, int i, uint32_t sh, uint32_t (&o)[4]) {
    const uint4 a = lds_read4(row + 4 * i);
    const uint32_t e = lds_read1(row + 4 * i + 16);
    o[0] = __builtin_amdgcn_alignbit(a.y, a.x, sh);
    o[1] = __builtin_amdgcn_alignbit(a.z, a.y, sh);
    o[2] = __builtin_amdgcn_alignbit(a.w, a.z, sh);
    o[3] = __builtin_amdgcn_alignbit(e, a.w, sh);
}

template <int NTOK, int N, int KH>
__device__ __forceinline__ void q6_quarter_run(const uint8_t* row, uint32_t sh, const uint32_t (&scw)[4],
                                               xconst_t xb, int64_t ldx, const float (&sx)[NTOK],
                                               float (&tl)[NTOK], float (&th)[NTOK]) {
    uint32_t A[4], B[4], H[4];
    q6_read4(row, 16 * N + 4 * KH, sh, A);          // ql bytes 64N + 16KH ..
    q6_read4(row, 16 * N + 8 + 4 * KH, sh, B);      // ql bytes 64N + 32 + 16KH ..
    q6_read4(row, 32 + 8 * N + 4 * KH, sh, H);      // qh bytes 32N + 16KH ..
    float a[4][NTOK];
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int t = 0; t < NTOK; ++t) a[c][t] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
        const int k = 4 * KH + kk;
        const Packed6 p = k6_codes(A[kk], B[kk], H[kk]);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int e = 128 * N + 32 * c + 4 * k;
#pragma unroll
            for (int t = 0; t < NTOK; ++t) {
                xconst_t xt = xb + t * ldx;
                a[c][t] = __builtin_fmaf((float)half_lo(p.c02[c]), xt[e + 0], a[c][t]);
                a[c][t] = __builtin_fmaf((float)half_lo(p.c13[c]), xt[e + 1], a[c][t]);
                a[c][t] = __builtin_fmaf((float)half_hi(p.c02[c]), xt[e + 2], a[c][t]);
                a[c][t] = __builtin_fmaf((float)half_hi(p.c13[c]), xt[e + 3], a[c][t]);
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int j = 8 * N + 2 * c + KH;                                   // sub-block of 16
        const float scj = (float)(int8_t)(scw[j / 4] >> (8 * (j % 4)));
        // code - 32: subtract 32*sum(x) in the units of a (2^-24 or 2^-20 per code)
        const float off = (c < 2) ? -0x1p-19f : -0x1p-15f;
#pragma unroll
        for (int t = 0; t < NTOK; ++t) {
            const float u = __builtin_fmaf(off, lane_value(sx[t], 4 * j), a[c][t]);
            if (c < 2) tl[t] = __builtin_fmaf(scj, u, tl[t]);
            else th[t] = __builtin_fmaf(scj, u, th[t]);
        }
    }
}

template <int NTOK>
__device__ __forceinline__ void item_q6(const KqDesc& T, const KqLaunch& L, const Item& it, uint8_t* slot) {
    const int lane = threadIdx.x;
    const uintptr_t tbase = reinterpret_cast<uintptr_t>(T.w) + (uintptr_t)it.r0 * T.row_bytes;
    const uintptr_t tend = reinterpret_cast<uintptr_t>(T.w) + (uintptr_t)T.rows * T.row_bytes;
    const bool word_lane = lane < kQ6Words;

    uint32_t stg[kTileRows];
#pragma unroll
    for (int r = 0; r < kTileRows; ++r) stg[r] = 0;
    // Row r of the column: 53 aligned words from the block start rounded down
    // to 4 bytes.  Only the tensor's very last block can end 2 bytes short of
    // its last word; that word is then read as 2 bytes.
    auto stage = [&](int b) {
#pragma unroll
        for (int r = 0; r < kTileRows; ++r) {
            if (r < it.rows_here) {
                const uintptr_t a = (tbase + (uintptr_t)r * T.row_bytes + 210u * (uintptr_t)b) & ~(uintptr_t)3;
                const uint8_t* p = reinterpret_cast<const uint8_t*>(a) + 4 * lane;
                if (a + 4 * kQ6Words <= tend) {
                    if (word_lane) stg[r] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
                } else {
                    if (lane < kQ6Words - 1) stg[r] = *reinterpret_cast<const uint32_t*>(p);
                    else if (lane == kQ6Words - 1) stg[r] = *reinterpret_cast<const uint16_t*>(p);
                }
            }
        }
    };

    float acc[NTOK];
#pragma unroll
    for (int t = 0; t < NTOK; ++t) acc[t] = 0.0f;
    const uint8_t* row = slot + lane * kQ6LdsRow;
    const bool even_nb = (T.nb & 1) == 0;

    stage(it.kb0);
    for (int b = it.kb0; b < it.kb1; ++b) {
        __syncthreads();
        if (word_lane) {
#pragma unroll
            for (int r = 0; r < kTileRows; ++r) reinterpret_cast<uint32_t*>(slot + r * kQ6LdsRow)[lane] = stg[r];
        }
        if (b + 1 < it.kb1) stage(b + 1);

        float sx[NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) sx[t] = subblock_sums<16>(T.x + t * T.ldx + 256 * b);

        __syncthreads();
        // the block starts 2 bytes into its first staged word when its index
        // in the tensor, (r0+lane)*nb + b, is odd
        const uint32_t sh = even_nb ? 16u * (uint32_t)(b & 1)
                                    : 16u * (uint32_t)(((int64_t)(it.r0 + lane) * T.nb + b) & 1);
        uint32_t scw[4];
        q6_read4(row, 48, sh, scw);
        const uint32_t dw = __builtin_amdgcn_alignbit(lds_read1(row + 4 * 53), lds_read1(row + 4 * 52), sh);
        const float d = f16_to_f32(dw & 0xFFFFu);
        xconst_t xb = (xconst_t)(T.x) + 256 * b;
        float tl[NTOK], th[NTOK];
#pragma unroll
        for (int t = 0; t < NTOK; ++t) { tl[t] = 0.0f; th[t] = 0.0f; }
        q6_quarter_run<NTOK, 0, 0>(row, sh, scw, xb, T.ldx, sx, tl, th);
        __builtin_amdgcn_sched_barrier(0);
        q6_quarter_run<NTOK, 0, 1>(row, sh, scw, xb, T.ldx, sx, tl, th);
        __builtin_amdgcn_sched_barrier(0);
        q6_quarter_run<NTOK, 1, 0>(row, sh, scw, xb, T.ldx, sx, tl, th);
        __builtin_amdgcn_sched_barrier(0);
        q6_quarter_run<NTOK, 1, 1>(row, sh, scw, xb, T.ldx, sx, tl, th);
        const float d24 = d * kTwo24;
#pragma unroll
        for (int t = 0; t < NTOK; ++t)
            acc[t] = __builtin_fmaf(d24, __builtin_fmaf(th[t], 0.0625f, tl[t]), acc[t]);
    }
    finish_item<NTOK>(T, L, it, acc);
}

// ------------------------------------------------------------ the kernel
template <int NTOK>
__global__ __launch_bounds__(64, (NTOK <= 7 ? 3 : 2)) void kq_matvec_kernel(const KqLaunch L) {
    extern __shared__ uint4 kq_slot[];
    const int item = xcd_item(blockIdx.x, gridDim.x);
    int ti = 0;
#pragma unroll 1
    for (int i = 1; i < L.n; ++i)
        if (item >= L.t[i].item_base) ti = i;
    const KqDesc& T = L.t[ti];
    const Item it = make_item(T, item - T.item_base);
    uint8_t* slot = reinterpret_cast<uint8_t*>(kq_slot);
    switch (T.fmt) {
    case KQ_Q4_K: item_k45<KQ_Q4_K, NTOK>(T, L, it, slot); break;
    case KQ_Q5_K: item_k45<KQ_Q5_K, NTOK>(T, L, it, slot); break;
    default: item_q6<NTOK>(T, L, it, slot); break;
    }
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

// ------------------------------------------------------------ launchers
int launch_matvec(const KqLaunch& L, hipStream_t stream) {
    dim3 grid(L.total_items), block(64);
    const size_t lds = (size_t)L.lds_bytes;
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
