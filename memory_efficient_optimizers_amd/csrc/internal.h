// Internal structures and device helpers of the optimizer-step library.
//
// Work decomposition:
//   * Apply-style passes cut a factored tensor, viewed as [B, H, W], into tiles of
//     kTileRows rows x kTileCols columns inside one matrix. A block of 256 threads
//     (4 wave64s) owns one tile: each lane owns 8 adjacent columns (one 16-byte
//     bf16 or two 16-byte fp32 accesses per row), each wave kRowsPerWave rows.
//   * The first (statistics) pass of a factored tensor whose rows fit a block
//     ("row-complete" tensors: 16-byte aligned, W % 8 == 0, W <= 12288) uses
//     strips of full rows (TDesc::srows of them): the block sees whole rows, so it finishes
//     the row statistic itself and can weight the column sums by it. Other
//     factored tensors use the 2-D tiles for their statistics too (and then need a
//     second read of G for the RMS of the update).
//   * A flat tensor (1-D Adafactor/CAME tensors, every LAMB tensor) is cut into
//     tiles of kFlatTile consecutive elements; each thread owns 8 adjacent
//     elements per iteration.
//   * Every launch reads a table of (tensor, tile-within-tensor) pairs, one per
//     block, built on the host for the whole tensor list.
// Every cross-block reduction is two-stage with a fixed order, so results are
// bitwise reproducible and independent of what else is in the list.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace meo {

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kLanes = 64;
constexpr int kVec = 8;                          // elements per lane per row/iteration
constexpr int kTileCols = kLanes * kVec;         // 512
constexpr int kRowsPerWave = 16;
constexpr int kTileRows = kWaves * kRowsPerWave; // 64
constexpr int kFlatIters = 16;
constexpr int kFlatTile = kThreads * kVec * kFlatIters;  // 32768
constexpr int kFinChunk = 256;                   // rows per finalize block
constexpr int kFinCols = 64;                     // columns per finalize block
constexpr int kScalSlots = 8;                    // floats of per-tensor scalars
// Rows per strip of the row-complete pass (TDesc::srows): 128 for Adafactor (half
// the column partials of 64-row strips; measured 1.6-2.5% faster steps on the 7B
// list), 64 for CAME.
constexpr int kStripRowsMax = 128;
constexpr int kStripRowsAdafactor = 128;
constexpr int kStripRowsCame = 64;
// Widest row of each row-complete class (class 0: 256 threads x 2 groups of 8
// columns; class 1: 512 threads x 3 groups).
constexpr int kRcMaxCols0 = 256 * 8 * 2;  // 4096
constexpr int kRcMaxCols1 = 512 * 8 * 3;  // 12288

// Per-tensor scalar slots in the workspace (their meaning is part of the C ABI:
// meo_*_scalar_offsets). LAMB keeps the parameter's norm in kSlotRmsX.
enum ScalSlot { kSlotAlpha = 0, kSlotCoef = 1, kSlotDecay = 2, kSlotRmsU = 3, kSlotRmsX = 4,
                kSlotNormD = 5, kSlotKappa = 6, kSlotTrust = 7 };

// Storage class of a launch's parameters and first moments: all fp32, all bf16,
// fp32 or bf16 parameters with 8-bit first moments, or a mix (then read per tensor
// from its descriptor). The streaming kernels are compiled once per class, so the
// uniform cases carry no dtype branches.
enum Storage { kStoreF32 = 0, kStoreBf16 = 1, kStoreMixed = 2, kStoreF32I8 = 3, kStoreBf16I8 = 4 };

// 8-bit first moment: one float32 scale per group of 128 consecutive values,
// i.e. 16 lanes of 8 values.
constexpr int kI8Group = 128;

// How a tensor's statistics are gathered.
enum Mode { kFlat = 0, kRowComplete = 1, kTiled = 2 };

// Device-side descriptor of one tensor of the call (built on the host, cached).
struct TDesc {
    void* x;          // parameter (fp32 or bf16)
    const void* g;    // gradient (fp32 or bf16)
    void* m;          // first moment (fp32, bf16 or int8 codes; nullable)
    float* ms;        // scales of an 8-bit first moment [ceil(numel / 128)]
    float* v;         // full second moment (1-D Adafactor/CAME; LAMB)
    float* r;         // factored row statistic [B*H]
    float* c;         // factored column statistic [B*W]
    float* rr;        // CAME confidence row statistic [B*H]
    float* rc;        // CAME confidence column statistic [B*W]
    int64_t numel;
    // workspace offsets, in floats
    int64_t rowpart;  // tiled: [B][tc][H] row sums per column tile
    int64_t colpart;  // tiled: [B][tr][W] column sums per row tile;
                      // row-complete: [B][strips][2][W] sums of Q and of G^2/R per strip
    int64_t sumr;     // tiled: [B][nrc] sums of the new row statistic per finalize chunk;
                      // row-complete: [B][ncc] sums of S_j / C_j per finalize chunk
    int64_t tilepart; // [tiles][2] per-tile partial sums for the per-tensor scalars
    int64_t xpart;    // row-complete: [xchunks] sums of X^2 per chunk of kFlatTile elements
    int64_t apart;    // Adafactor: [tiles] sums of the updated X^2 per apply tile (carried sum(X^2))
    float* xsq;       // Adafactor: the carried sum(X^2) of the parameter [1] (nullable)
    int64_t bscal;    // [2][B] per-matrix coefficients
    int64_t scal;     // [kScalSlots] per-tensor scalars
    int32_t B, H, W;
    int32_t mode;     // Mode
    int32_t gbf16;    // gradient dtype is bf16
    int32_t xbf16;    // parameter dtype is bf16
    int32_t mbf16;    // first-moment dtype is bf16
    int32_t mi8;      // first moment is 8-bit group-quantized
    int32_t vec;      // 16-byte vector accesses are valid
    int32_t tr, tc;   // 2-D tiles per matrix along rows / columns (flat: tr = 1, tc = tiles)
    int32_t strips;   // row-complete strips per matrix
    int32_t srows;    // rows per row-complete strip
    int32_t nrc, ncc; // finalize chunks per matrix along rows / columns
    int32_t xchunks;  // row-complete: chunks of the parameter for sum(X^2)
    // Row-sharded steps: where the tensor's record starts in the partial-sum buffer
    // (floats) and the size of the whole tensor (rows of each matrix when factored,
    // elements when flat).
    int64_t part;
    int64_t total;
    int64_t part2;    // CAME: the tensor's record of confidence sums (second exchange)
};

// One launch: its (tensor, local tile) items and the shared descriptors.
struct Table {
    const TDesc* desc;
    const int2* items;  // [grid] x = tensor index, y = tile (or finalize item) within the tensor;
                        // in the row-complete first pass y < 0 marks chunk -1 - y of sum(X^2);
                        // x < 0: an empty item (padding of an XCD-aligned streaming list)
    float* ws;          // workspace base
};

// ----------------------------------------------------------------------------- helpers

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Element types of a tensor's parameter and first moment under storage class ST.
template <int ST>
__device__ __forceinline__ bool x_is_bf16(const TDesc& d) {
    return ST == kStoreMixed ? d.xbf16 != 0 : (ST == kStoreBf16 || ST == kStoreBf16I8);
}
template <int ST>
__device__ __forceinline__ bool m_is_bf16(const TDesc& d) {
    return ST == kStoreMixed ? d.mbf16 != 0 : ST == kStoreBf16;
}
template <int ST>
__device__ __forceinline__ bool m_is_i8(const TDesc& d) {
    return ST == kStoreMixed ? d.mi8 != 0 : (ST == kStoreF32I8 || ST == kStoreBf16I8);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Sum over the block (NW waves) of two per-thread values, in a fixed order;
// result valid in thread 0. `lds` holds 2 * NW floats.
template <int NW = kWaves>
__device__ __forceinline__ void block_sum2(float& a, float& b, float* lds) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    a = wave_sum(a);
    b = wave_sum(b);
    if (lane == 0) { lds[w] = a; lds[NW + w] = b; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float sa = lds[0], sb = lds[NW];
#pragma unroll
        for (int i = 1; i < NW; ++i) { sa += lds[i]; sb += lds[NW + i]; }
        a = sa;
        b = sb;
    }
}

__device__ __forceinline__ double block_sum_d(double a, double* lds) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    a = wave_sum(a);
    if (lane == 0) lds[w] = a;
    __syncthreads();
    return (lds[0] + lds[1]) + (lds[2] + lds[3]);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Pointers read from the launch table are generic; every tensor lives in device
// global memory, so accesses go through address-space-1 pointers (global_load /
// global_store instead of flat_*).
#define MEO_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const MEO_GLOBAL T* gld(const void* p) {
    return (const MEO_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ MEO_GLOBAL T* gst(void* p) {
    return (MEO_GLOBAL T*)(p);
}

// 16-byte loads; NT marks data read once (non-temporal hint).
template <bool NT>
__device__ __forceinline__ u32x4 ld_u4(const void* p) {
    if (NT) return __builtin_nontemporal_load(gld<u32x4>(p));
    return *gld<u32x4>(p);
}
template <bool NT>
__device__ __forceinline__ f32x4 ld_f4(const void* p) {
    if (NT) return __builtin_nontemporal_load(gld<f32x4>(p));
    return *gld<f32x4>(p);
}

__device__ __forceinline__ void bf16x8(const u32x4 u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

// 8 values starting at element `i` of the fp32 or bf16 tensor `g` (gradient,
// parameter or first moment), widened to fp32; `valid` (0..8) of them are in range,
// the rest read as 0. Vector loads only when all 8 are valid and `vec`.
template <bool NT = false>
__device__ __forceinline__ void load_v8(const void* __restrict__ g, int64_t i, int valid,
                                        bool vec, bool bf16, float* f) {
    if (bf16) {
        const uint16_t* p = static_cast<const uint16_t*>(g) + i;
        if (vec && valid == kVec) {
            bf16x8(ld_u4<NT>(p), f);
        } else {
            const MEO_GLOBAL uint16_t* q = gld<uint16_t>(p);
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                f[e] = e < valid ? __uint_as_float(static_cast<uint32_t>(q[e]) << 16) : 0.0f;
        }
    } else {
        const float* p = static_cast<const float*>(g) + i;
        if (vec && valid == kVec) {
            const f32x4 a = ld_f4<NT>(p);
            const f32x4 b = ld_f4<NT>(p + 4);
            f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
            f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
        } else {
            const MEO_GLOBAL float* q = gld<float>(p);
#pragma unroll
            for (int e = 0; e < kVec; ++e) f[e] = e < valid ? q[e] : 0.0f;
        }
    }
}

template <bool NT = false>
__device__ __forceinline__ void load_f8(const float* __restrict__ p, int valid, bool vec, float* f) {
    if (vec && valid == kVec) {
        const f32x4 a = ld_f4<NT>(p);
        const f32x4 b = ld_f4<NT>(p + 4);
        f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
        f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
    } else {
        const MEO_GLOBAL float* q = gld<float>(p);
#pragma unroll
        for (int e = 0; e < kVec; ++e) f[e] = e < valid ? q[e] : 0.0f;
    }
}

__device__ __forceinline__ void store_f8(float* __restrict__ p, int valid, bool vec, const float* f) {
    if (vec && valid == kVec) {
        *gst<f32x4>(p) = f32x4{f[0], f[1], f[2], f[3]};
        *gst<f32x4>(p + 4) = f32x4{f[4], f[5], f[6], f[7]};
    } else {
        MEO_GLOBAL float* q = gst<float>(p);
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e < valid) q[e] = f[e];
    }
}

// Nearest bf16 value of f (ties to even; NaN stays NaN), as fp32.
__device__ __forceinline__ float round_bf16(float f) {
    return static_cast<float>(static_cast<__bf16>(f));
}

__device__ __forceinline__ uint32_t bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}


// 8 fp32 values rounded to bf16 (nearest, ties to even), packed in element order.
__device__ __forceinline__ u32x4 pack_bf16x8(const float* f) {
    return u32x4{bf16_bits(f[0]) | (bf16_bits(f[1]) << 16), bf16_bits(f[2]) | (bf16_bits(f[3]) << 16),
                 bf16_bits(f[4]) | (bf16_bits(f[5]) << 16), bf16_bits(f[6]) | (bf16_bits(f[7]) << 16)};
}

// Stores 8 fp32 values at element `i` of the fp32 or bf16 tensor `p`, bf16 rounded
// to nearest (ties to even); only the first `valid` are written.
__device__ __forceinline__ void store_v8(void* __restrict__ p, int64_t i, int valid, bool vec, bool bf16,
                                         const float* f) {
    if (bf16) {
        uint16_t* q = static_cast<uint16_t*>(p) + i;
        if (vec && valid == kVec) {
            *gst<u32x4>(q) = pack_bf16x8(f);
        } else {
            MEO_GLOBAL uint16_t* s = gst<uint16_t>(q);
#pragma unroll
            for (int e = 0; e < kVec; ++e)
                if (e < valid) s[e] = static_cast<uint16_t>(bf16_bits(f[e]));
        }
    } else {
        store_f8(static_cast<float*>(p) + i, valid, vec, f);
    }
}

// Buffer resources: a base address and a byte range held in scalar registers, so a
// wave addresses rows of a tile with one 32-bit lane offset plus a scalar row
// offset instead of a 64-bit address per lane and row. Accesses beyond
// `bytes` read 0 and write nothing.
typedef __amdgpu_buffer_rsrc_t Rsrc;
__device__ __forceinline__ Rsrc make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ u32x4 buf_ld(Rsrc r, uint32_t lane_off, uint32_t row_off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, row_off, 0);
}
__device__ __forceinline__ void buf_st(u32x4 v, Rsrc r, uint32_t lane_off, uint32_t row_off) {
    __builtin_amdgcn_raw_buffer_store_b128(v, r, lane_off, row_off, 0);
}

// ----------------------------------------------------------------------------- 8-bit first moment

// 8 values of an 8-bit first moment at element i (a multiple of 8): codes times
// their group's scale, in fp32; the `valid` first are in range, the rest read 0.
__device__ __forceinline__ void load_i8x8(const void* __restrict__ codes, const float* __restrict__ scales,
                                          int64_t i, int valid, bool vec, float* f) {
    if (valid <= 0) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) f[e] = 0.0f;
        return;
    }
    const float s = *gld<float>(scales + (i >> 7));
    const int8_t* p = static_cast<const int8_t*>(codes) + i;
    if (vec && valid == kVec) {
        typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
        const u32x2v w = *gld<u32x2v>(p);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            f[e] = static_cast<float>(static_cast<int8_t>(w.x >> (8 * e))) * s;
            f[4 + e] = static_cast<float>(static_cast<int8_t>(w.y >> (8 * e))) * s;
        }
    } else {
        const MEO_GLOBAL int8_t* q = gld<int8_t>(p);
#pragma unroll
        for (int e = 0; e < kVec; ++e) f[e] = e < valid ? static_cast<float>(q[e]) * s : 0.0f;
    }
}

// Re-quantizes this lane's 8 new values together with the 15 other lanes of its
// group of 128 (lanes 16k..16k+15 hold consecutive values): scale = max|m| / 127,
// code = m / scale rounded half to even and clamped to [-128, 127] (0 when the
// scale is 0; a NaN or infinite maximum gives scale NaN and codes 0). `m` is
// replaced by the dequantized values. Values outside the tensor must be 0. Every
// lane of the wave calls it (cross-lane maximum).
// Larger of two magnitudes, a NaN winning.
__device__ __forceinline__ float max_nan(float a, float b) { return (b > a || b != b) ? b : a; }

// DPP move within a row of 16 lanes (all lanes active).
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

__device__ __forceinline__ void quant_i8x8(float* m, uint32_t& lo, uint32_t& hi, float& scale) {
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < kVec; ++e) a = max_nan(a, fabsf(m[e]));
    // Maximum over the 16 lanes of the group, which is one DPP row: swap neighbours,
    // swap pairs, mirror halves, mirror the row.
    a = max_nan(a, dpp<0xb1>(a));   // quad_perm [1, 0, 3, 2]
    a = max_nan(a, dpp<0x4e>(a));   // quad_perm [2, 3, 0, 1]
    a = max_nan(a, dpp<0x141>(a));  // row_half_mirror
    a = max_nan(a, dpp<0x140>(a));  // row_mirror
    scale = a / 127.0f;
    const bool ok = scale > 0.0f && scale <= 3.402823466e38f;  // finite and nonzero
    if (!(scale <= 3.402823466e38f)) scale = __builtin_nanf("");
    lo = 0u;
    hi = 0u;
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        float q = ok ? rintf(m[e] / scale) : 0.0f;  // the fp32 quotient, rounded half to even
        q = fminf(fmaxf(q, -128.0f), 127.0f);
        const uint32_t byte = static_cast<uint32_t>(static_cast<int32_t>(q)) & 0xffu;
        if (e < 4) lo |= byte << (8 * e); else hi |= byte << (8 * (e - 4));
        m[e] = q * scale;  // a zero scale reads back 0, a NaN one NaN
    }
}

// Stores the codes of quant_i8x8 at element i (the `valid` first of 8) and, from
// the first lane of each group that holds data, the group's scale.
__device__ __forceinline__ void store_i8x8(void* __restrict__ codes, float* __restrict__ scales, int64_t i,
                                           int valid, bool vec, uint32_t lo, uint32_t hi, float scale) {
    if (valid <= 0) return;
    int8_t* p = static_cast<int8_t*>(codes) + i;
    if (vec && valid == kVec) {
        typedef unsigned int u32x2v __attribute__((ext_vector_type(2)));
        *gst<u32x2v>(p) = u32x2v{lo, hi};
    } else {
        MEO_GLOBAL int8_t* q = gst<int8_t>(p);
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            if (e < valid) q[e] = static_cast<int8_t>(((e < 4 ? lo >> (8 * e) : hi >> (8 * (e - 4)))) & 0xffu);
    }
    if ((i & (kI8Group - 1)) == 0) *gst<float>(scales + (i >> 7)) = scale;
}

// Storage of a new first moment: bf16 rounding or 8-bit re-quantization (with
// its codes and scale kept for the store). After settle_m8, `m` holds the values
// the rest of the step uses; every lane of the wave calls it.
struct Q8 {
    uint32_t lo = 0u, hi = 0u;
    float s = 0.0f;
};
__device__ __forceinline__ void load_m8(const TDesc& d, int64_t i, int valid, bool vec, bool mb, bool mi, float* f) {
    if (mi) load_i8x8(d.m, d.ms, i, valid, vec, f);
    else load_v8(d.m, i, valid, vec, mb, f);
}
__device__ __forceinline__ void settle_m8(float* m, bool mb, bool mi, Q8& q) {
    if (mi) {
        quant_i8x8(m, q.lo, q.hi, q.s);
    } else if (mb) {
#pragma unroll
        for (int e = 0; e < kVec; ++e) m[e] = round_bf16(m[e]);
    }
}
__device__ __forceinline__ void store_m8(const TDesc& d, int64_t i, int valid, bool vec, bool mb, bool mi,
                                         const float* m, const Q8& q) {
    if (mi) store_i8x8(d.m, d.ms, i, valid, vec, q.lo, q.hi, q.s);
    else store_v8(d.m, i, valid, vec, mb, m);
}

// Scalar accesses of state vectors and workspace through generic pointers.
__device__ __forceinline__ float ldf(const float* p) { return *gld<float>(p); }
__device__ __forceinline__ void stf(float* p, float v) { *gst<float>(p) = v; }

__device__ __forceinline__ int clamp_valid(int64_t remaining) {
    return remaining >= kVec ? kVec : (remaining > 0 ? static_cast<int>(remaining) : 0);
}

__device__ __forceinline__ float sum8(const float* a) {
    return ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
}

// ----------------------------------------------------------------------------- tile helpers

// Mean over the rows of matrix b of the (already updated) row statistic of a
// tiled tensor, from the per-chunk sums written by the finalize pass. Every lane of
// the calling wave gets the same value, and every caller the same bits.
__device__ __forceinline__ double row_mean_tiled(const TDesc& d, const float* __restrict__ ws, int b) {
    const int lane = threadIdx.x & 63;
    const float* sr = ws + d.sumr + static_cast<int64_t>(b) * d.nrc;
    double s = 0.0;
    for (int j = lane; j < d.nrc; j += kLanes) s += static_cast<double>(ldf(sr + j));
    return wave_sum(s) / static_cast<double>(d.H);
}

// The same for a row-complete tensor, whose strips summed their new row statistic.
__device__ __forceinline__ double row_mean_rc(const TDesc& d, const float* __restrict__ ws, int b) {
    const int lane = threadIdx.x & 63;
    const float* tp = ws + d.tilepart + 2 * static_cast<int64_t>(b) * d.strips;
    double s = 0.0;
    for (int j = lane; j < d.strips; j += kLanes) s += static_cast<double>(ldf(tp + 2 * j));
    return wave_sum(s) / static_cast<double>(d.H);
}

struct TileRC {   // this thread's position inside a 2-D tile
    int b, rt, ct, col, valid, row0, nrows;
};

__device__ __forceinline__ TileRC tile_rc(const TDesc& d, int lt) {
    TileRC p;
    const int per = d.tr * d.tc;
    p.b = lt / per;
    const int rem = lt - p.b * per;
    p.rt = rem / d.tc;
    p.ct = rem - p.rt * d.tc;
    const int w = uniform(threadIdx.x >> 6), lane = threadIdx.x & 63;
    p.col = p.ct * kTileCols + lane * kVec;
    p.valid = clamp_valid(static_cast<int64_t>(d.W) - p.col);
    p.row0 = p.rt * kTileRows + w * kRowsPerWave;
    p.nrows = min(kRowsPerWave, d.H - p.row0);
    return p;
}

// Column partial sums of one 2-D tile: the 4 waves' per-lane sums are combined in
// a fixed order through LDS (kWaves * kTileCols floats) and written to
// colpart[b][rt][col].
__device__ __forceinline__ void write_colpart(const TDesc& d, float* __restrict__ ws, const TileRC& p,
                                              const float* cs, float* lds) {
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    float* l = lds + w * kTileCols + lane * kVec;
    *reinterpret_cast<float4*>(l) = make_float4(cs[0], cs[1], cs[2], cs[3]);
    *reinterpret_cast<float4*>(l + 4) = make_float4(cs[4], cs[5], cs[6], cs[7]);
    __syncthreads();
    float* out = ws + d.colpart + (static_cast<int64_t>(p.b) * d.tr + p.rt) * d.W;
    for (int cc = threadIdx.x; cc < kTileCols; cc += kThreads) {
        const int cg = p.ct * kTileCols + cc;
        if (cg < d.W)
            stf(out + cg, (lds[cc] + lds[kTileCols + cc]) + (lds[2 * kTileCols + cc] + lds[3 * kTileCols + cc]));
    }
}

// ----------------------------------------------------------------------------- launchers

// Arguments of the shared passes.
struct StatsArgs {      // statistics of Q = G^2 + eps1
    float eps1;
    float beta;         // EMA weight of the old statistic (beta2t or beta2); 0: not read
    float omb;          // 1 - beta, rounded from fp64
    int32_t need_x;     // also accumulate sum(x^2)
    double dbeta;       // the same weights in fp64 (row statistic of row-complete strips)
    double domb;
};
struct FinArgs {        // row/column finalize: s <- beta*s + (1-beta)*mean(partials)
    double beta;        // 0: the old statistic is not read
    int32_t which;      // 0: squared-gradient statistic (r, c); 1: CAME confidence (rr, rc)
    int32_t tiled_all;  // 1: every factored tensor has tiled partials (CAME's second statistic)
};
enum ScalMode { kScalAdafactor = 0, kScalCame1 = 1, kScalCame2 = 2, kScalLamb = 3 };
struct ScalArgs {
    int32_t mode;
    int32_t scale_parameter;
    const float* partials;  // row-sharded steps: the all-reduced partial sums; else null
    int32_t carried_x;      // Adafactor: take sum(X^2) from each tensor's carried value (TDesc::xsq)
    double rho;         // Adafactor base step size
    double eps2;        // Adafactor floor of RMS(param)
    double clip;        // clip threshold
    double wd;          // weight decay
    double lr;          // CAME / LAMB learning rate
};
struct AfApplyArgs {
    float beta1, omb1;
    int32_t has_beta1;
};
struct CameArgs {
    float beta1, omb1;
    float eps2;
    float lr;
};
struct LambArgs {
    float beta1, omb1, beta2, omb2;
    float inv_bc1, inv_bc2;  // 1 / (1 - beta^t), or 1 without bias correction
    float eps, wd;
};

// Row-complete first pass, class 0 (W <= 4096, also the flat tensors' first pass)
// and class 1 (W <= 12288).
void launch_rowstats(int cls, const Table& t, int64_t n, const StatsArgs& a, hipStream_t s);
void launch_xnorm(const Table& t, int64_t n, const StatsArgs& a, hipStream_t s);
void launch_stats(const Table& t, int64_t n, const StatsArgs& a, hipStream_t s);
void launch_finalize(const Table& t, int64_t n, const FinArgs& a, hipStream_t s);
void launch_rms(const Table& t, int64_t n, int32_t need_x, hipStream_t s);
void launch_scalars(const TDesc* desc, float* ws, int32_t n, const ScalArgs& a, hipStream_t s);
// sumsq: also sum the squares of the updated parameter per tile (into TDesc::apart).
void launch_af_apply(const Table& t, int64_t n, const AfApplyArgs& a, int storage, bool sumsq, hipStream_t s);
// Folds the per-tile sums of the updated X^2 into each tensor's carried value.
void launch_sumsq_fold(const TDesc* desc, const float* ws, int32_t n, hipStream_t s);
void launch_came_mom(const Table& t, int64_t n, const CameArgs& a, int storage, hipStream_t s);
void launch_came_apply(const Table& t, int64_t n, int storage, hipStream_t s);
void launch_lamb_moments(const Table& t, int64_t n, const LambArgs& a, int storage, hipStream_t s);
void launch_lamb_apply(const Table& t, int64_t n, const LambArgs& a, int storage, hipStream_t s);
// Row-sharded steps: the shard's partial sums, and their fold (after the caller's
// all-reduce) into the replicated column statistic.
// carried (Adafactor): the sum of X^2 comes from each tensor's carried value.
void launch_shard_partials(const Table& t, int64_t n, float* partials, int32_t need_x, int32_t carried,
                           hipStream_t s);
void launch_shard_fold(const Table& t, int64_t n, const float* partials, double beta, hipStream_t s);
// Zero-fills records (x = first float, y = length) of tensors a rank holds none of.
void launch_zero_records(const int2* items, int64_t n, float* partials, hipStream_t s);
// CAME's second exchange: the shard's column sums of the instability and the sum
// of its new confidence row statistic; then their fold into the replicated
// confidence column statistic.
void launch_conf_partials(const Table& t, int64_t n, float* conf, hipStream_t s);
void launch_conf_fold(const Table& t, int64_t n, const float* conf, double beta, hipStream_t s);

}  // namespace meo
