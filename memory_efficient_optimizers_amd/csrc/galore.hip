// GaLore step on matrix cores. The Colossal-AI distributed-optimizers page (section
// on GaLore's special configuration) describes a projector that keeps an
// orthogonal matrix, refreshed by an SVD every update_proj_gap steps: project()
// turns the full-rank gradient into a low-rank one on which the optimizer (AdamW)
// runs, and project_back() multiplies the low-rank update by `scale` and restores
// the full shape. With proj_type "std" the projection is along the shorter side
// (the rank / min(m, n) state compression the page states):
//
//   m >= n: R = G U          (U: n x r)     update = scale * N U^T
//   m <  n: R^T = G^T U      (U: m x r)     update = scale * U N^T
//
// so the low-rank arrays are always [max(m, n)][r]. Two kernels per step:
//
//   k_galore_project_mixed / k_galore_project_wide / k_galore_project
//                     R = X U with X = G (m >= n) or G^T (m < n), bf16 MFMA with
//                     fp32 accumulation, one 256-row (wide) or 64-row tile of R
//                     per block and the whole contraction in the block (no split
//                     partials); the epilogue runs AdamW on the tile: moments updated in place,
//                     direction N = m_hat / (sqrt(v_hat) + eps) written as two
//                     bf16 planes (high part and the remainder) so that the back
//                     projection keeps ~16 significant bits of N on bf16 MFMA.
//   k_galore_back_ur / k_galore_back_u2 / k_galore_back
//                     W <- W (1 - lr wd) - lr scale (N U^T or U N^T): two bf16
//                     MFMAs per fragment (high and low plane), the parameter tile
//                     read and written once; the U-register kernels keep a 256-row
//                     block of U in registers and walk up to 4096 rows of N
//                     (k_galore_back_u2: bf16 parameters, m >= n, two 4-wave
//                     blocks per CU).
//
// The projector is kept in bf16 (the gradient's type) both as U [d][r] and as
// U^T [r][d], so every operand is read with the contraction index contiguous.
// The only transposed read is G in the m < n projection: the wide kernel stages
// G's rows as they lie and reads them with the LDS transpose read; the
// register-staged kernel scatters them transposed into LDS. Non-projected
// tensors take a flat AdamW kernel (k_galore_adamw).
#include "galore.h"

#include <type_traits>

namespace meo {

typedef __bf16 bfv8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma32(const bfv8& a, const bfv8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 8 bf16 (raw bits) of row `row` starting at column `col` of a row-major [rows][cols]
// array; out-of-range elements read 0.
__device__ __forceinline__ u32x4 ld_row8(const uint16_t* p, int64_t rows, int64_t cols, int64_t row,
                                         int64_t col, bool vec) {
    if (row >= rows || col >= cols) return u32x4{0u, 0u, 0u, 0u};
    const uint16_t* q = p + row * cols + col;
    if (vec && col + 8 <= cols) return *gld<u32x4>(q);
    const MEO_GLOBAL uint16_t* s = gld<uint16_t>(q);
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const uint32_t lo = col + 2 * e < cols ? s[2 * e] : 0u;
        const uint32_t hi = col + 2 * e + 1 < cols ? s[2 * e + 1] : 0u;
        w[e] = lo | (hi << 16);
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

__device__ __forceinline__ void st_lds8(uint16_t* p, const u32x4& v) {
    *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bfv8 ld_frag(const uint16_t* p) {
    return *reinterpret_cast<const bfv8*>(p);
}

// Rows [r0, r0 + NROWS) x contraction columns [k0, k0 + kGaKb) of a row-major
// [rows][cols] bf16 array, zero outside it: loaded into registers first (all of a
// thread's chunks in flight at once, and the next block's while the current one
// is multiplied), then written to LDS (row pitch kGaPitch).
template <int NROWS, int THREADS = kThreads>
struct RowStage {
    static constexpr int kPer = NROWS * (kGaKb / 8) / THREADS;
    u32x4 v[kPer];
    __device__ __forceinline__ void load(const uint16_t* p, int64_t rows, int64_t cols, int64_t r0, int64_t k0,
                                         bool vec) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * THREADS;
            v[i] = ld_row8(p, rows, cols, r0 + (c >> 3), k0 + (c & 7) * 8, vec);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * THREADS;
            st_lds8(lds + (c >> 3) * kGaPitch + (c & 7) * 8, v[i]);
        }
    }
};

// The transposed tile A[i][k] = G[k0 + k][i0 + i] (i < kGaTile, k < kGaKb) of the
// row-major gradient G [K][D]: loaded along G's rows, scattered into LDS.
template <int IROWS>
struct TransStage {
    static constexpr int kRowChunks = IROWS / 8;  // 16-byte chunks per row of G
    static constexpr int kPer = kGaKb * kRowChunks / kThreads;
    u32x4 v[kPer];
    __device__ __forceinline__ void load(const uint16_t* g, int64_t K, int64_t D, int64_t i0, int64_t k0, bool vec) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            v[i] = ld_row8(g, K, D, k0 + c / kRowChunks, i0 + (c % kRowChunks) * 8, vec);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int k = c / kRowChunks, ic = (c % kRowChunks) * 8;
            const uint32_t w[4] = {v[i].x, v[i].y, v[i].z, v[i].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                lds[(ic + 2 * e) * kGaPitch + k] = static_cast<uint16_t>(w[e] & 0xffffu);
                lds[(ic + 2 * e + 1) * kGaPitch + k] = static_cast<uint16_t>(w[e] >> 16);
            }
        }
    }
};

// Accumulator element v of a 32x32 block held by `lane`: row and column in the block.
__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }
__device__ __forceinline__ int acc_col(int lane) { return lane & 31; }

// Epilogue exchange: a wave's 32 x 64 half tile (accumulator blocks (ib, 0) and
// (ib, 1)) goes through LDS so that each lane then holds 8 consecutive columns
// of a row, for 16-byte loads and stores of the row-major outputs. Lane l gets
// rows (l >> 3) + 8 q (q < 4) and columns 8 (l & 7) .. 8 (l & 7) + 7. Only the
// wave itself touches its LDS region, and its LDS accesses run in program order.
constexpr int kEpPitch = 68;  // floats per LDS row of the exchange
constexpr int kEpWave = 32 * kEpPitch;

__device__ __forceinline__ void ep_spill(const f32x16& a0, const f32x16& a1, float* lw, int lane) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
        lw[acc_row(v, lane) * kEpPitch + (lane & 31)] = a0[v];
        lw[acc_row(v, lane) * kEpPitch + 32 + (lane & 31)] = a1[v];
    }
    __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ void ep_gather(const float* lw, int lane, int q, float* c) {
    const float* p = lw + ((lane >> 3) + 8 * q) * kEpPitch + (lane & 7) * 8;
    const f32x4 x0 = *reinterpret_cast<const f32x4*>(p);
    const f32x4 x1 = *reinterpret_cast<const f32x4*>(p + 4);
    c[0] = x0.x; c[1] = x0.y; c[2] = x0.z; c[3] = x0.w;
    c[4] = x1.x; c[5] = x1.y; c[6] = x1.z; c[7] = x1.w;
    __builtin_amdgcn_wave_barrier();
}

// ------------------------------------------------------------------ projection + AdamW

// Direct staging: rows of 64 bf16 (128 bytes, unpadded) written straight from
// global memory into LDS by global_load_lds (no registers), 8 rows per
// instruction: lane l fills row (l >> 3) of the group at 16-byte slot (l & 7),
// which holds the row's chunk (l & 7) ^ sw_row(row). A fragment read (16 lanes per
// LDS cycle on 64 banks: 16 consecutive rows, one chunk each) then finds rows r and
// r + 8 on different slots as well as the 8 rows of each parity: no bank conflict
// (with sw_row(r) = r & 7 alone rows r and r + 8 collided, which doubled the LDS
// cycles of the projection). Rows past the operand's end read its last row: they
// only reach outputs that are not stored.
constexpr int kDirectPitch = kGaKb;  // bf16 per LDS row
__device__ __forceinline__ int sw_row(int r) { return (r & 7) ^ ((r >> 3) & 1); }
template <int ROWS, int THREADS = kThreads>
__device__ __forceinline__ void stage_direct(const uint16_t* g, int64_t nrows, int64_t cols, int64_t r0, int k0,
                                             uint16_t* dst, int wave, int lane) {
#pragma unroll
    for (int j = wave; j < ROWS / 8; j += THREADS / 64) {
        const int rr = 8 * j + (lane >> 3);
        const int64_t row = min(r0 + rr, nrows - 1);
        const int c = (lane & 7) ^ sw_row(rr);
        const uint16_t* src = g + row * cols + k0 + c * 8;
        __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)src,
                                         (__attribute__((address_space(3))) void*)(dst + 8 * j * kDirectPitch),
                                         16, 0, 0);
    }
}

__device__ __forceinline__ bfv8 ld_frag_sw(const uint16_t* base, int row, int kk) {
    return *reinterpret_cast<const bfv8*>(base + row * kDirectPitch + (((kk >> 3) ^ sw_row(row)) << 3));
}


__device__ __forceinline__ void galore_adamw8(const GDesc& d, const GaArgs& a, int64_t row, int col, const float* rv) {
    float m[8], v[8], nh[8], nl[8];
    const int64_t idx = row * d.r + col;
    const bool full = d.rvec && col + 8 <= d.r;
    if (full) {
        const f32x4 m0 = *gld<f32x4>(d.em + idx), m1 = *gld<f32x4>(d.em + idx + 4);
        const f32x4 v0 = *gld<f32x4>(d.ev + idx), v1 = *gld<f32x4>(d.ev + idx + 4);
        m[0] = m0.x; m[1] = m0.y; m[2] = m0.z; m[3] = m0.w; m[4] = m1.x; m[5] = m1.y; m[6] = m1.z; m[7] = m1.w;
        v[0] = v0.x; v[1] = v0.y; v[2] = v0.z; v[3] = v0.w; v[4] = v1.x; v[5] = v1.y; v[6] = v1.z; v[7] = v1.w;
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            m[e] = col + e < d.r ? *gld<float>(d.em + idx + e) : 0.0f;
            v[e] = col + e < d.r ? *gld<float>(d.ev + idx + e) : 0.0f;
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        m[e] = fmaf(a.beta1, m[e], a.omb1 * rv[e]);
        v[e] = fmaf(a.beta2, v[e], a.omb2 * (rv[e] * rv[e]));
        const float n = (m[e] * a.inv_bc1) / (sqrtf(v[e] * a.inv_bc2) + a.eps);
        nh[e] = round_bf16(n);
        nl[e] = n - nh[e];
    }
    if (full) {
        *gst<f32x4>(d.em + idx) = f32x4{m[0], m[1], m[2], m[3]};
        *gst<f32x4>(d.em + idx + 4) = f32x4{m[4], m[5], m[6], m[7]};
        *gst<f32x4>(d.ev + idx) = f32x4{v[0], v[1], v[2], v[3]};
        *gst<f32x4>(d.ev + idx + 4) = f32x4{v[4], v[5], v[6], v[7]};
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < d.r) {
                *gst<float>(d.em + idx + e) = m[e];
                *gst<float>(d.ev + idx + e) = v[e];
            }
    }
    if (d.vec && col + 8 <= d.r) {  // the planes are 256-byte aligned; rows of r % 8 == 0
        *gst<u32x4>(d.nh + idx) = pack_bf16x8(nh);
        *gst<u32x4>(d.nl + idx) = pack_bf16x8(nl);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (col + e < d.r) {
                *gst<uint16_t>(d.nh + idx + e) = static_cast<uint16_t>(bf16_bits(nh[e]));
                *gst<uint16_t>(d.nl + idx + e) = static_cast<uint16_t>(bf16_bits(nl[e]));
            }
    }
}

// Register-staged projection, for lists the wide kernel does not take (a
// contraction length that is not a multiple of kGaKb, or rows without 16-byte
// alignment). Tile: kGaProjRows rows of R x all r columns; wave w holds columns
// 64w .. 64w + 63. With 64-row tiles, 3 waves per SIMD.
template <bool Left>
__global__ __launch_bounds__(kThreads, kGaProjRB == 1 ? 3 : 2) void k_galore_project(GTable t, GaArgs a) {
    constexpr int kRB = 2 * kGaProjRB;  // 32-row blocks of a wave's tile
    constexpr int kPitch = kGaPitch;
    __shared__ __attribute__((aligned(16))) uint16_t arena[(kGaProjRows + kGaWide) * kPitch];
    static_assert((kGaProjRows + kGaWide) * kPitch * 2 >= kWaves * kEpWave * 4, "exchange space");
    uint16_t* sa = arena;
    uint16_t* sb = arena + kGaProjRows * kPitch;
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of the XCD-dealt list (the whole block)
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i0 = static_cast<int64_t>(it.y) * kGaProjRows;
    const bool vec = d.vec, active = wave * 64 < d.r;
    f32x16 acc[kRB][2];
#pragma unroll
    for (int ib = 0; ib < kRB; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.0f;

    typename std::conditional<Left, TransStage<kGaProjRows>, RowStage<kGaProjRows>>::type pa;
    RowStage<kGaWide> pb;
    auto fetch = [&](int64_t k0) {
        if constexpr (Left) pa.load(d.g, d.d, d.D, i0, k0, vec);
        else pa.load(d.g, d.D, d.d, i0, k0, vec);
        pb.load(d.ut, d.r, d.d, 0, k0, vec);
    };
    auto multiply = [&]() {
        if (!active) return;
#pragma unroll
        for (int ks = 0; ks < kGaKb; ks += 16) {
            const int kk = ks + 8 * (lane >> 5);
            bfv8 fa[kRB], fb[2];
#pragma unroll
            for (int ib = 0; ib < kRB; ++ib) fa[ib] = ld_frag(sa + (ib * 32 + (lane & 31)) * kGaPitch + kk);
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) fb[jb] = ld_frag(sb + (wave * 64 + jb * 32 + (lane & 31)) * kGaPitch + kk);
#pragma unroll
            for (int ib = 0; ib < kRB; ++ib)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma32(fa[ib], fb[jb], acc[ib][jb]);
        }
    };
    fetch(0);
    for (int64_t k0 = 0; k0 < d.d; k0 += kGaKb) {
        pa.store(sa);
        pb.store(sb);
        __syncthreads();
        if (k0 + kGaKb < d.d) fetch(k0 + kGaKb);
        multiply();
        __syncthreads();
    }
    if (!active) return;
    // AdamW on the tile of R, rows of 8 columns per lane (see ep_spill): moments
    // read and written, N's planes written, 16 bytes at a time where rows allow.
    float* lw = reinterpret_cast<float*>(arena) + wave * kEpWave;
#pragma unroll
    for (int ib = 0; ib < kRB; ++ib) {
        ep_spill(acc[ib][0], acc[ib][1], lw, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = i0 + ib * 32 + (lane >> 3) + 8 * q;
            const int col = wave * 64 + (lane & 7) * 8;
            if (row >= d.D || col >= d.r) continue;
            float rv[8];
            ep_gather(lw, lane, q, rv);
            galore_adamw8(d, a, row, col, rv);
        }
    }
}


// Wide projection (lists whose contraction length is a multiple of kGaKb and
// whose rows allow 16-byte loads): a 256-row x r tile of R per block of 8 waves,
// wave w at rows 128 (w / 4) and columns 64 (w % 4), one block per CU. The G and
// U^T blocks of one contraction step (64 long) go by global_load_lds into one of
// two LDS stages (separate arrays, so that the compiler tells the stages apart and
// waits only for the stage being read): step k + 1 is in flight while step k is
// multiplied. Every wave issues exactly kPwDma transfers per stage, so waiting
// until at most kPwDma are outstanding means the older stage has landed. Against
// the 64-row tile of k_galore_project, each U^T block serves 4x the rows: its L2
// reads per row drop 4x, and the projection of the Llama-7B-shaped list ran
// 6.32 -> 5.11 ms (both sides), with bitwise the same results.
constexpr int kPwDma = 2 * kGaPwRows / 8 / (kGaPwThreads / 64);   // 8
// One stage: the G block and the U^T block of the contraction step at k0 (64
// columns of the contraction each), 256 rows each, by global_load_lds.
//   m >= n: G rows i0 .. i0 + 255 (rows of R), contraction along G's rows: the
//           swizzled 64-column layout that ld_frag_sw reads.
//   m < n:  G rows k0 .. k0 + 63 (the contraction runs down G's columns),
//           columns i0 .. i0 + 255 (rows of R): 64 LDS rows of 256 (512 bytes),
//           whose 16-byte chunk c sits at position c ^ (4 (row & 3)); instruction j
//           fills rows 2j and 2j + 1. ld_frag_tr reads it transposed.
template <bool Left>
__device__ __forceinline__ void pw_stage(const GDesc& d, int64_t i0, int k0, uint16_t* sa, uint16_t* sb, int wave,
                                         int lane) {
#pragma unroll
    for (int i = 0; i < kGaPwRows / 8 / (kGaPwThreads / 64); ++i) {
        const int j = wave + i * (kGaPwThreads / 64);
        const int rr = 8 * j + (lane >> 3);
        const int c = (lane & 7) ^ sw_row(rr);
        if constexpr (Left) {
            const int kr = 2 * j + (lane >> 5);
            const int64_t cc = min(i0 / 8 + ((lane & 31) ^ ((kr & 3) << 2)), static_cast<int64_t>(d.D) / 8 - 1);
            __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)(d.g + (k0 + kr) * static_cast<int64_t>(d.D) + cc * 8),
                                             (__attribute__((address_space(3))) void*)(sa + j * 512), 16, 0, 0);
        } else {
            const int64_t ra = min(i0 + rr, static_cast<int64_t>(d.D) - 1);
            __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)(d.g + ra * d.d + k0 + c * 8),
                                             (__attribute__((address_space(3))) void*)(sa + 8 * j * kDirectPitch), 16, 0, 0);
        }
        const int64_t rb = min(rr, d.r - 1);
        __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)(d.ut + rb * d.d + k0 + c * 8),
                                         (__attribute__((address_space(3))) void*)(sb + 8 * j * kDirectPitch), 16, 0, 0);
    }
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));

// MFMA A fragment of rows r0 .. r0 + 31 of R at contraction offset ks from the
// transposed G stage (m < n), by LDS transpose reads: within each 16-lane group the
// read hands lane i the i-th 16-bit element of each of the 4 rows that lanes
// 4e + (i >> 2) address, so lanes 4e + q point at row kbase + e, columns
// cbase + 4q .. + 3 and lane i receives column cbase + i at rows kbase .. kbase + 3.
// Lane l (group g = l >> 4) gets row r0 + (l & 31) at contraction rows
// ks + 8 (l >> 5) .. + 7, as the MFMA wants; two reads give the 8.
__device__ __forceinline__ bfv8 ld_frag_tr(const uint16_t* sa, int r0, int ks, int lane) {
    const int g = lane >> 4, e = (lane >> 2) & 3, q = lane & 3;
    const int col = r0 + 16 * (g & 1) + 4 * q;
    const int kr = ks + 8 * (g >> 1) + e;
    const int off = (((col >> 3) ^ (e << 2)) << 3) + (col & 7);  // (kr & 3) == e for both reads
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(sa + kr * 256 + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(sa + (kr + 4) * 256 + off));
    const s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bfv8, v);
}

// s_waitcnt with only the vector-memory count (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their no-wait maxima).
#define MEO_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | (7 << 4) | (15 << 8))

// One 256-row tile of R (rows i0 ..) of tensor d: the contraction through the two
// LDS stages (a0/b0, a1/b1: the kernel's own arrays, so that the compiler tells
// the stages apart), then AdamW on the tile.
template <bool Left>
__device__ __forceinline__ void pw_tile(const GDesc& d, int64_t i0, const GaArgs& a, uint16_t* a0, uint16_t* b0,
                                        uint16_t* a1, uint16_t* b1) {
    static_assert(kPwDma == 8, "wait counts below");
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int rg = wave >> 2, cg = wave & 3;
    const bool active = cg * 64 < d.r;
    f32x16 acc[4][2];
#pragma unroll
    for (int ib = 0; ib < 4; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.0f;
    // Fragments of sub-step ks + 16 are read while sub-step ks is multiplied.
    auto multiply = [&](const uint16_t* sa, const uint16_t* sb) {
        if (!active) return;
        bfv8 fa[2][4], fb[2][2];
        auto load = [&](int ks, int buf) {
            const int kk = ks + 8 * (lane >> 5);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib) {
                if constexpr (Left) fa[buf][ib] = ld_frag_tr(sa, rg * 128 + ib * 32, ks, lane);
                else fa[buf][ib] = ld_frag_sw(sa, rg * 128 + ib * 32 + (lane & 31), kk);
            }
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) fb[buf][jb] = ld_frag_sw(sb, cg * 64 + jb * 32 + (lane & 31), kk);
        };
        load(0, 0);
#pragma unroll
        for (int s4 = 0; s4 < kGaKb / 16; ++s4) {
            if (s4 + 1 < kGaKb / 16) load((s4 + 1) * 16, (s4 + 1) & 1);
#pragma unroll
            for (int ib = 0; ib < 4; ++ib)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma32(fa[s4 & 1][ib], fb[s4 & 1][jb], acc[ib][jb]);
        }
        // Schedule (the compiler otherwise waits for each sub-step's reads before its
        // MFMAs, leaving the SIMD idle): the first sub-step's LDS reads, then each
        // later sub-step's reads one by one between the 8 MFMAs of the current one
        // (m < n: 10 reads, two transpose reads per A fragment; the last two follow
        // the MFMAs). Right side, Llama-7B list: 3.95 -> 3.75 ms.
        constexpr int kReads = Left ? 10 : 6;
        constexpr int kPaired = kReads < 8 ? kReads : 8;
        __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);  // 0x100: LDS reads
#pragma unroll
        for (int s4 = 0; s4 + 1 < kGaKb / 16; ++s4) {
#pragma unroll
            for (int r = 0; r < kPaired; ++r) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            }
            if (8 > kPaired) __builtin_amdgcn_sched_group_barrier(0x008, 8 - kPaired, 0);
            if (kReads > kPaired) __builtin_amdgcn_sched_group_barrier(0x100, kReads - kPaired, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    };
    // Every stage issues its transfers unconditionally (past the last step it
    // fetches the last block again), so that each wait below is the same count.
    const int nk = d.d / kGaKb, last = nk - 1;
    pw_stage<Left>(d, i0, 0, a0, b0, wave, lane);
    pw_stage<Left>(d, i0, min(1, last) * kGaKb, a1, b1, wave, lane);
    MEO_WAIT_VM(8);
    __builtin_amdgcn_s_barrier();
    multiply(a0, b0);
    __builtin_amdgcn_s_barrier();
    for (int kb = 1; kb < nk; kb += 2) {
        pw_stage<Left>(d, i0, min(kb + 1, last) * kGaKb, a0, b0, wave, lane);  // stage 1 holds step kb
        MEO_WAIT_VM(8);
        __builtin_amdgcn_s_barrier();
        multiply(a1, b1);
        __builtin_amdgcn_s_barrier();
        if (kb + 1 >= nk) break;
        pw_stage<Left>(d, i0, min(kb + 2, last) * kGaKb, a1, b1, wave, lane);  // stage 0 holds step kb + 1
        MEO_WAIT_VM(8);
        __builtin_amdgcn_s_barrier();
        multiply(a0, b0);
        __builtin_amdgcn_s_barrier();
    }
    MEO_WAIT_VM(0);  // every wave's last, repeated transfers land before the LDS is reused
    __builtin_amdgcn_s_barrier();
    if (!active) return;
    uint16_t* ex = wave < 3 ? a0 : (wave < 6 ? b0 : a1);
    float* lw = reinterpret_cast<float*>(ex) + (wave % 3) * kEpWave;
#pragma unroll
    for (int ib = 0; ib < 4; ++ib) {
        ep_spill(acc[ib][0], acc[ib][1], lw, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = i0 + rg * 128 + ib * 32 + (lane >> 3) + 8 * q;
            const int col = cg * 64 + (lane & 7) * 8;
            if (row >= d.D || col >= d.r) continue;
            float rv[8];
            ep_gather(lw, lane, q, rv);
            galore_adamw8(d, a, row, col, rv);
        }
    }
}

template <bool Left>
__global__ __launch_bounds__(kGaPwThreads, 1) void k_galore_project_wide(GTable t, GaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t a0[kGaPwRows * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t b0[kGaWide * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t a1[kGaPwRows * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t b1[kGaWide * kDirectPitch];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;
    pw_tile<Left>(t.desc[it.x], static_cast<int64_t>(it.y) * kGaPwRows, a, a0, b0, a1, b1);
}

// Both sides' tiles in one launch: descriptors [0, nright) are right-side ones (the
// side follows proj_type, not only the shape). A launch leaves part of its last round
// of blocks idle; one launch instead of two has one such tail (Llama-7B list at rank
// 256: 5.05 -> 4.99 ms for the projection, results bitwise the same).
__global__ __launch_bounds__(kGaPwThreads, 1) void k_galore_project_mixed(GTable t, GaArgs a, int nright) {
    __shared__ __attribute__((aligned(16))) uint16_t a0[kGaPwRows * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t b0[kGaWide * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t a1[kGaPwRows * kDirectPitch];
    __shared__ __attribute__((aligned(16))) uint16_t b1[kGaWide * kDirectPitch];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;
    const GDesc d = t.desc[it.x];
    const int64_t i0 = static_cast<int64_t>(it.y) * kGaPwRows;
    if (it.x >= nright) pw_tile<true>(d, i0, a, a0, b0, a1, b1);
    else pw_tile<false>(d, i0, a, a0, b0, a1, b1);
}

void launch_galore_project_mixed(const GTable& t, int64_t n, int nright, const GaArgs& a, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_galore_project_mixed, dim3(static_cast<uint32_t>(n)), dim3(kGaPwThreads), 0, s, t, a,
                       nright);
}

void launch_galore_project(const GTable& t, int64_t n, const GaArgs& a, bool left, bool direct, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (direct && left) hipLaunchKernelGGL((k_galore_project_wide<true>), grid, dim3(kGaPwThreads), 0, s, t, a);
    else if (direct) hipLaunchKernelGGL((k_galore_project_wide<false>), grid, dim3(kGaPwThreads), 0, s, t, a);
    else if (left) hipLaunchKernelGGL(k_galore_project<true>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_galore_project<false>, grid, block, 0, s, t, a);
}

// ------------------------------------------------------------------ back-projection + update

// Tiles of W: 64 kGaBackRW rows x 256 columns for m >= n (C = Nh U^T + Nl U^T),
// 256 rows x 64 kGaBackRW columns for m < n (C = U Nh^T + U Nl^T); 4 kGaBackRW
// waves of 64 x 64, wave w at U group w % 4 and N group w / 4. A larger tile
// shares each staged U block among more rows of N: per output element the staging
// reads 4r / 256 + 2r / (64 kGaBackRW) bytes from L2.
constexpr int kBackThreads = kThreads * kGaBackRW;
constexpr int kBackN = kGaTile * kGaBackRW;  // rows of N per tile

// Direct: operands staged by global_load_lds into an unpadded swizzled arena
// (48 KB: 3 blocks per CU), for lists whose rank is a multiple of kGaKb; otherwise
// through registers into a padded arena (55 KB) with the next block's loads in
// flight during the multiply.
template <bool Left, bool Direct>
__global__ __launch_bounds__(kBackThreads, Direct ? 3 : 1) void k_galore_back(GTable t, GaArgs a) {
    // one arena: N's planes [kBackN][pitch] twice, then U [256][pitch]; reused by
    // the epilogue exchange (4 kGaBackRW x 8.5 KB)
    constexpr int kPitch = Direct ? kDirectPitch : kGaPitch;
    __shared__ __attribute__((aligned(16))) uint16_t arena[(2 * kBackN + kGaWide) * kPitch];
    static_assert((2 * kBackN + kGaWide) * kPitch * 2 >= kBackThreads / 64 * kEpWave * 4, "exchange space");
    uint16_t* sh = arena;                         // N, high plane
    uint16_t* sl = arena + kBackN * kPitch;       // N, low plane
    uint16_t* su = arena + 2 * kBackN * kPitch;   // U rows
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of the XCD-dealt list
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ug = wave & 3, ng = wave >> 2;  // the wave's 64-row groups of U and of N
    const int ti = it.y / d.btj, tj = it.y % d.btj;
    // Tile origin in W; the N side indexes N's rows, the 256-wide side U's rows.
    const int64_t r0 = Left ? static_cast<int64_t>(ti) * kGaWide : static_cast<int64_t>(ti) * kBackN;
    const int64_t c0 = Left ? static_cast<int64_t>(tj) * kBackN : static_cast<int64_t>(tj) * kGaWide;
    const int64_t n0 = Left ? c0 : r0;  // first row of N in the tile
    const int64_t u0 = Left ? r0 : c0;  // first row of U in the tile
    const bool vec = d.vec;
    f32x16 acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.0f;

    RowStage<kBackN, kBackThreads> ph, pl;
    RowStage<kGaWide, kBackThreads> pu;
    auto fetch = [&](int k0) {
        ph.load(d.nh, d.D, d.r, n0, k0, vec);
        pl.load(d.nl, d.D, d.r, n0, k0, vec);
        pu.load(d.u, d.d, d.r, u0, k0, vec);
    };
    // The wave's part of the parameter tile, as the epilogue reads it (lane: rows
    // (lane >> 3) + 8 q of each 32-row half ib, columns 8 (lane & 7) ..): loaded
    // during the last contraction block, when the staging registers are free, so
    // that its HBM latency overlaps those MFMAs. Chunks that are not whole 16-byte
    // rows are read in the epilogue instead.
    const int64_t wr0 = Left ? r0 + ug * 64 : r0 + ng * 64;
    const int64_t wc0 = Left ? c0 + ng * 64 : c0 + ug * 64;
    const int64_t wcol = wc0 + (lane & 7) * 8;
    // Direct: only the first 16 rows of the wave's tile (16 VGPRs for fp32), which
    // is what the registers left at 3 blocks per CU hold without spilling.
    constexpr int kDirectPreQ = 2;
    auto pre = [](int ib, int q) { return !Direct || (ib == 0 && q < kDirectPreQ); };
    u32x4 wpre[2][4][2];
    auto prefetch_w = [&]() {
        if (!(d.wvec && wcol + 8 <= d.n)) return;
#pragma unroll
        for (int ib = 0; ib < 2; ++ib)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t row = wr0 + ib * 32 + (lane >> 3) + 8 * q;
                if (!pre(ib, q) || row >= d.m) continue;
                const int64_t idx = row * d.n + wcol;
                if (d.xbf16) {
                    wpre[ib][q][0] = *gld<u32x4>(static_cast<const uint16_t*>(d.x) + idx);
                } else {
                    wpre[ib][q][0] = *gld<u32x4>(static_cast<const float*>(d.x) + idx);
                    wpre[ib][q][1] = *gld<u32x4>(static_cast<const float*>(d.x) + idx + 4);
                }
            }
    };
    // One staged contraction block: 4 steps of 16, two MFMAs (high and low plane)
    // per accumulator block.
    auto multiply = [&]() {
#pragma unroll
        for (int ks = 0; ks < kGaKb; ks += 16) {
            const int kk = ks + 8 * (lane >> 5);
            bfv8 fu[2], fh[2], fl[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                if constexpr (Direct) {
                    fu[b] = ld_frag_sw(su, ug * 64 + b * 32 + (lane & 31), kk);
                    fh[b] = ld_frag_sw(sh, ng * 64 + b * 32 + (lane & 31), kk);
                    fl[b] = ld_frag_sw(sl, ng * 64 + b * 32 + (lane & 31), kk);
                } else {
                    fu[b] = ld_frag(su + (ug * 64 + b * 32 + (lane & 31)) * kGaPitch + kk);
                    fh[b] = ld_frag(sh + (ng * 64 + b * 32 + (lane & 31)) * kGaPitch + kk);
                    fl[b] = ld_frag(sl + (ng * 64 + b * 32 + (lane & 31)) * kGaPitch + kk);
                }
            }
#pragma unroll
            for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                for (int jb = 0; jb < 2; ++jb) {
                    if (Left) {  // rows from U, columns from N
                        acc[ib][jb] = mfma32(fu[ib], fh[jb], acc[ib][jb]);
                        acc[ib][jb] = mfma32(fu[ib], fl[jb], acc[ib][jb]);
                    } else {     // rows from N, columns from U
                        acc[ib][jb] = mfma32(fh[ib], fu[jb], acc[ib][jb]);
                        acc[ib][jb] = mfma32(fl[ib], fu[jb], acc[ib][jb]);
                    }
                }
        }
    };
    const int klast = (d.r - 1) / kGaKb * kGaKb;
    if constexpr (Direct) {
        // the rank is a multiple of kGaKb: every contraction block is whole
        for (int k0 = 0; k0 <= klast; k0 += kGaKb) {
            stage_direct<kBackN, kBackThreads>(d.nh, d.D, d.r, n0, k0, sh, wave, lane);
            stage_direct<kBackN, kBackThreads>(d.nl, d.D, d.r, n0, k0, sl, wave, lane);
            stage_direct<kGaWide, kBackThreads>(d.u, d.d, d.r, u0, k0, su, wave, lane);
            __syncthreads();  // the loads have landed (each wave waits for its own first)
            if (k0 == klast) prefetch_w();
            multiply();
            __syncthreads();
        }
    } else {
    fetch(0);
    // All blocks but the last: the next block's loads go out before the multiply.
    // The last one (peeled, so that the parameter registers are live only there
    // and in the epilogue) prefetches the parameter tile instead.
    for (int k0 = 0; k0 < klast; k0 += kGaKb) {
        ph.store(sh);
        pl.store(sl);
        pu.store(su);
        __syncthreads();
        fetch(k0 + kGaKb);
        multiply();
        __syncthreads();
    }
    ph.store(sh);
    pl.store(sl);
    pu.store(su);
    __syncthreads();
    prefetch_w();
    multiply();
    __syncthreads();
    }
    // W <- decay W - coef C, rows of 8 columns per lane (see ep_spill), 16 bytes at
    // a time where rows allow.
    float* lw = reinterpret_cast<float*>(arena) + wave * kEpWave;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib) {
        // The row groups not prefetched are all loaded before any is stored (a store
        // may alias a later load as far as the compiler knows).
        u32x4 wl[4][2];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = wr0 + ib * 32 + (lane >> 3) + 8 * q;
            if (pre(ib, q) || !(d.wvec && wcol + 8 <= d.n) || row >= d.m) continue;
            const int64_t idx = row * d.n + wcol;
            if (d.xbf16) {
                wl[q][0] = *gld<u32x4>(static_cast<const uint16_t*>(d.x) + idx);
            } else {
                wl[q][0] = *gld<u32x4>(static_cast<const float*>(d.x) + idx);
                wl[q][1] = *gld<u32x4>(static_cast<const float*>(d.x) + idx + 4);
            }
        }
        ep_spill(acc[ib][0], acc[ib][1], lw, lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int64_t row = wr0 + ib * 32 + (lane >> 3) + 8 * q;
            const int64_t col = wc0 + (lane & 7) * 8;
            if (row >= d.m || col >= d.n) continue;
            float c[8], w[8];
            ep_gather(lw, lane, q, c);
            const int64_t idx = row * d.n + col;
            const bool full = d.wvec && col + 8 <= d.n;
            if (d.xbf16) {
                uint16_t* xp = static_cast<uint16_t*>(d.x) + idx;
                if (full) {
                    bf16x8(pre(ib, q) ? wpre[ib][q][0] : wl[q][0], w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        w[e] = col + e < d.n ? __uint_as_float(static_cast<uint32_t>(*gld<uint16_t>(xp + e)) << 16) : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = a.decay * w[e] - a.coef * c[e];
                if (full) {
                    *gst<u32x4>(xp) = pack_bf16x8(w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < d.n) *gst<uint16_t>(xp + e) = static_cast<uint16_t>(bf16_bits(w[e]));
                }
            } else {
                float* xp = static_cast<float*>(d.x) + idx;
                if (full) {
                    const u32x4 x0 = pre(ib, q) ? wpre[ib][q][0] : wl[q][0];
                    const u32x4 x1 = pre(ib, q) ? wpre[ib][q][1] : wl[q][1];
                    w[0] = __uint_as_float(x0.x); w[1] = __uint_as_float(x0.y);
                    w[2] = __uint_as_float(x0.z); w[3] = __uint_as_float(x0.w);
                    w[4] = __uint_as_float(x1.x); w[5] = __uint_as_float(x1.y);
                    w[6] = __uint_as_float(x1.z); w[7] = __uint_as_float(x1.w);
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = col + e < d.n ? *gld<float>(xp + e) : 0.0f;
                }
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = a.decay * w[e] - a.coef * c[e];
                if (full) {
                    *gst<f32x4>(xp) = f32x4{w[0], w[1], w[2], w[3]};
                    *gst<f32x4>(xp + 4) = f32x4{w[4], w[5], w[6], w[7]};
                } else {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if (col + e < d.n) *gst<float>(xp + e) = w[e];
                }
            }
        }
    }
}


// Back-projection with the U block in registers (lists whose rank is a multiple of
// kGaKb and whose rows allow 16-byte loads). An item is 256 rows of U (a band of W's
// columns for m >= n, of its rows for m < n) and up to kUrTiles consecutive 64-row
// tiles of N. The block's 8 waves (wave w: U rows 32 w, all 64 rows of a tile's N)
// load their U fragments for the whole rank once, 64 VGPRs; then per tile
// only N's planes are staged, by global_load_lds, into one of two LDS buffers (64 KB
// each: rows of 256, chunk c of row w at c ^ (w & 15)), the next tile's while the
// current one is multiplied. The parameter part of tile i + 1 is loaded right after
// tile i's stores and the next stage, so it has tile i + 1's contraction to land; the
// wait before a tile leaves exactly those stores, that stage and those loads
// outstanding. Against the direct-staged 64 x 256 tiles (3 blocks per CU, U staged
// per tile) the L2 bytes staged per tile fall from 192 KB to 64 KB: Llama-7B list,
// fp32 parameters, 13.55 -> 12.57 ms (bf16 10.2 -> 9.95 ms), results bitwise the
// same. The parameter stream (one read and one write of W) bounds it: timing-only
// copies take 10.8 ms with the parameter stream alone in these tiles (5.0 TB/s), and
// the same with the products but N staged once; each tile's N stage is what the pass
// spends beyond that.
constexpr int kUrN = kGaTile;           // rows of N per tile
constexpr int kUrNDma = 2 * kUrN * (kGaWide / 8) / 64 / 8;  // 16-byte transfers per wave per tile: 8
// A wave's 32 x 32 exchange block in LDS, unpadded: row r at row r ^ ((r >> 2) & 1), its
// 16-byte chunk c at chunk c ^ ((r >> 1) & 1), so that neither the accumulator spill
// (rows r and r + 4 at once) nor the 8-column gather (rows 4k .. 4k + 3) hits a bank twice.
__device__ __forceinline__ int ur_ex(int r, int col) {
    return ((r ^ ((r >> 2) & 1)) << 5) + ((((col >> 2) ^ ((r >> 1) & 1))) << 2) + (col & 3);
}

__device__ __forceinline__ void ur_stage(const GDesc& d, int64_t n0, uint16_t* buf, int wave, int lane) {
    // instruction j: rows 2j, 2j + 1 of one plane (plane = j / 32), 32 chunks each
#pragma unroll
    for (int i = 0; i < kUrNDma; ++i) {
        const int j = wave + 8 * i;                 // 0 .. 63
        const int plane = j >> 5, jr = j & 31;
        const int row = 2 * jr + (lane >> 5);       // 0 .. 63
        const int c = (lane & 31) ^ (row & 15);     // global chunk held at position lane & 31
        const int cc = min(c, d.r / 8 - 1);
        const int64_t grow = min(n0 + row, static_cast<int64_t>(d.D) - 1);
        const uint16_t* src = (plane ? d.nl : d.nh) + grow * d.r + cc * 8;
        __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)src,
                                         (__attribute__((address_space(3))) void*)(buf + j * 512), 16, 0, 0);
    }
}

__device__ __forceinline__ bfv8 ur_frag(const uint16_t* plane, int row, int kk) {
    return *reinterpret_cast<const bfv8*>(plane + row * 256 + ((((kk >> 3) ^ (row & 15))) << 3));
}

template <bool Left, bool XB>
__global__ __launch_bounds__(512, 1) void k_galore_back_ur(GTable t, GaArgs a) {
    static_assert(kUrNDma == 8, "wait counts below");
    constexpr int kP = XB ? 4 : 8;  // 16-byte parameter loads (and stores) per lane per tile
    __shared__ __attribute__((aligned(16))) uint16_t nb0[2 * kUrN * 256];
    __shared__ __attribute__((aligned(16))) uint16_t nb1[2 * kUrN * 256];
    __shared__ __attribute__((aligned(16))) float exb[8 * 32 * 32];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of the XCD-dealt list
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nc = d.btj;  // chunks of kUrTiles tiles per band
    const int band = it.y / nc, chunk = it.y % nc;
    const int64_t u0 = static_cast<int64_t>(band) * kGaWide;
    const int64_t nt0 = static_cast<int64_t>(chunk) * kUrTiles;
    const int ntiles = static_cast<int>(min<int64_t>(kUrTiles, (d.D + kUrN - 1) / kUrN - nt0));
    const int nks = d.r / 16;  // 16-wide contraction sub-steps
    using PT = typename std::conditional<XB, uint16_t, float>::type;
    PT* const x = static_cast<PT*>(d.x);
    // U fragments of the wave's 32 rows for the whole rank (64 VGPRs), landed before the
    // pipeline starts so that no wait inside it has to cover them
    bfv8 uf[16];
    {
        const int64_t row = min(u0 + wave * 32 + (lane & 31), static_cast<int64_t>(d.d) - 1);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int k = min(ks, nks - 1) * 16 + 8 * (lane >> 5);
            uf[ks] = __builtin_bit_cast(bfv8, *gld<u32x4>(d.u + row * d.r + k));
        }
    }
    MEO_WAIT_VM(0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) __asm__ volatile("" : "+v"(uf[ks]));
    // W cells of the wave: two 32 x 32 blocks (blk: the tile's 32-row halves of N); in
    // block blk, lane holds rows (lane >> 2) + 16 q (q < 2), columns 8 (lane & 3) .. + 7.
    auto cell = [&](int64_t n0, int blk, int q, int64_t& row, int64_t& col) {
        const int r = (lane >> 2) + 16 * q, c = 8 * (lane & 3);
        if (Left) {  // rows from U, columns from N
            row = u0 + wave * 32 + r;
            col = n0 + blk * 32 + c;
        } else {     // rows from N, columns from U
            row = n0 + blk * 32 + r;
            col = u0 + wave * 32 + c;
        }
    };
    u32x4 wp[2][2][2];  // [block][q][16-byte half]
    // exactly kP loads, rows and columns clamped into the tensor
    auto load_w = [&](int64_t n0) {
        if (!d.wvec) return;  // only the exact path (16-byte rows) uses them
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                int64_t row, col;
                cell(n0, blk, q, row, col);
                row = min(row, static_cast<int64_t>(d.m) - 1);
                col = min(col, static_cast<int64_t>(d.n) - 8);
                const PT* p = x + row * d.n + col;
                wp[blk][q][0] = *gld<u32x4>(p);
                if (!XB) wp[blk][q][1] = *gld<u32x4>(p + 4);
            }
    };
    f32x16 acc[2];
    auto multiply = [&](const uint16_t* buf) {
        const uint16_t* ph = buf;
        const uint16_t* pl = buf + kUrN * 256;
        // The fragment reads are one asm block per sub-step that waits for its own
        // reads: the compiler cannot tell which stage an LDS read hits, and before a
        // plain read it would wait for every outstanding transfer, the next stage and
        // the parameter loads included. The stage read here landed (the wait and the
        // barrier before the multiply).
        // One address per sub-step: the low plane is 32 KB on, rows r + 32 are 16 KB on
        // (same swizzle, since r + 32 = r mod 16).
        static_assert(kUrN * 256 * 2 == 32768, "plane offset in the reads below");
        (void)pl;
        const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(ph)) + (lane & 31) * 512;
        const int sw = lane & 15;
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            if (ks >= nks) break;
            const int kc = 2 * ks + (lane >> 5);  // 16-byte chunk of the row
            int swv = sw;
            __asm__ volatile("" : "+v"(swv));  // computed here, not hoisted and spilled
            const uint32_t addr = base + static_cast<uint32_t>((kc ^ swv) << 4);
            u32x4 h0, l0, h1, l1;
            __asm__ volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %4 offset:32768\n\t"
                "ds_read_b128 %2, %4 offset:16384\n\t"
                "ds_read_b128 %3, %4 offset:49152\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(h0), "=&v"(l0), "=&v"(h1), "=&v"(l1)
                : "v"(addr));
            const bfv8 fh[2] = {__builtin_bit_cast(bfv8, h0), __builtin_bit_cast(bfv8, h1)};
            const bfv8 fl[2] = {__builtin_bit_cast(bfv8, l0), __builtin_bit_cast(bfv8, l1)};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                if (Left) {
                    acc[b] = mfma32(uf[ks], fh[b], acc[b]);
                    acc[b] = mfma32(uf[ks], fl[b], acc[b]);
                } else {
                    acc[b] = mfma32(fh[b], uf[ks], acc[b]);
                    acc[b] = mfma32(fl[b], uf[ks], acc[b]);
                }
            }
        }
    };
    // W <- decay W - coef C for a tile, through the wave's exchange region (one 32 x 32
    // block at a time, so that each lane ends with 8 consecutive columns of a row).
    // exact: every cell inside the tensor, exactly kP 16-byte stores; otherwise
    // element-wise edges and a full wait after them.
    auto update = [&](int64_t n0, bool exact) {
        float* lw = exb + wave * (32 * 32);
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
#pragma unroll
            for (int v = 0; v < 16; ++v) lw[ur_ex(acc_row(v, lane), acc_col(lane))] = acc[blk][v];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float cq[8];
                {
                    const int r = (lane >> 2) + 16 * q, c = 8 * (lane & 3);
                    const f32x4 c0 = *reinterpret_cast<const f32x4*>(lw + ur_ex(r, c));
                    const f32x4 c1 = *reinterpret_cast<const f32x4*>(lw + ur_ex(r, c + 4));
                    cq[0] = c0.x; cq[1] = c0.y; cq[2] = c0.z; cq[3] = c0.w;
                    cq[4] = c1.x; cq[5] = c1.y; cq[6] = c1.z; cq[7] = c1.w;
                }
                int64_t row, col;
                cell(n0, blk, q, row, col);
                float w[8];
                if (exact) {
                    PT* xp = x + row * d.n + col;
                    if (XB) {
                        bf16x8(wp[blk][q][0], w);
                    } else {
                        const u32x4 x0 = wp[blk][q][0], x1 = wp[blk][q][1];
                        w[0] = __uint_as_float(x0.x); w[1] = __uint_as_float(x0.y);
                        w[2] = __uint_as_float(x0.z); w[3] = __uint_as_float(x0.w);
                        w[4] = __uint_as_float(x1.x); w[5] = __uint_as_float(x1.y);
                        w[6] = __uint_as_float(x1.z); w[7] = __uint_as_float(x1.w);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = a.decay * w[e] - a.coef * cq[e];
                    if (XB) {
                        *gst<u32x4>(xp) = pack_bf16x8(w);
                    } else {
                        *gst<f32x4>(xp) = f32x4{w[0], w[1], w[2], w[3]};
                        *gst<f32x4>(xp + 4) = f32x4{w[4], w[5], w[6], w[7]};
                    }
                } else {
                    if (row >= d.m || col >= d.n) continue;
                    PT* xp = x + row * d.n + col;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (col + e >= d.n) continue;
                        const float w0 = XB ? __uint_as_float(static_cast<uint32_t>(*gld<uint16_t>(reinterpret_cast<const uint16_t*>(xp) + e)) << 16)
                                            : *gld<float>(reinterpret_cast<const float*>(xp) + e);
                        const float w1 = a.decay * w0 - a.coef * cq[e];
                        if (XB) *gst<uint16_t>(reinterpret_cast<uint16_t*>(xp) + e) = static_cast<uint16_t>(bf16_bits(w1));
                        else *gst<float>(reinterpret_cast<float*>(xp) + e) = w1;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();  // this block's gathers before the next block's spill
        }
        if (!exact) MEO_WAIT_VM(0);
    };
    auto zero = [&]() {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;
    };
    // Exact counts need every tile of the item whole and 16-byte parameter rows.
    const bool exact = d.wvec && (nt0 + ntiles) * kUrN <= d.D && u0 + kGaWide <= d.d;
    // Tile i uses buffer i & 1. After tile i's update, the stage for tile i + 2 goes
    // out (past the last tile it stages the last one again, so counts stay fixed), then
    // the parameter loads of tile i + 1. So the loads are the newest transfers: the
    // update of tile i + 1, whose first use of them makes the compiler wait for every
    // transfer in flight, waits for them and for older ones only, not for a stage
    // issued after them (with the loads before the stage, that wait covered the stage:
    // 12.43 -> 12.06 ms for the fp32 back-projection of the Llama-7B list, bf16 9.80
    // -> 9.35 ms, results bitwise the same). The wait before a tile's products allows
    // 2 kP + 8 transfers in flight, all issued after that tile's stage: the previous
    // tile's kP stores, the next stage's 8 transfers and this tile's kP loads (before
    // the first tile: the next stage's 8 and its kP loads, or no loads where the
    // parameter rows are not 16-byte aligned and load_w issues none).
    const int last = ntiles - 1;
    ur_stage(d, nt0 * kUrN, nb0, wave, lane);
    ur_stage(d, (nt0 + min(1, last)) * kUrN, nb1, wave, lane);
    load_w(nt0 * kUrN);
    if (d.wvec) MEO_WAIT_VM(kP + 8);
    else MEO_WAIT_VM(8);
    for (int i = 0; i < ntiles; i += 2) {
        // tile i in nb0 (its stage landed)
        __builtin_amdgcn_s_barrier();
        zero();
        multiply(nb0);
        __builtin_amdgcn_s_barrier();
        update((nt0 + i) * kUrN, exact);
        if (i + 1 >= ntiles) break;
        // tile i + 1 in nb1
        ur_stage(d, (nt0 + min(i + 2, last)) * kUrN, nb0, wave, lane);
        load_w((nt0 + i + 1) * kUrN);
        if (exact) MEO_WAIT_VM(2 * kP + 8);
        else MEO_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        zero();
        multiply(nb1);
        __builtin_amdgcn_s_barrier();
        update((nt0 + i + 1) * kUrN, exact);
        if (i + 2 >= ntiles) break;
        ur_stage(d, (nt0 + min(i + 3, last)) * kUrN, nb1, wave, lane);
        load_w((nt0 + i + 2) * kUrN);
        if (exact) MEO_WAIT_VM(2 * kP + 8);
        else MEO_WAIT_VM(0);
    }
    MEO_WAIT_VM(0);
}

// m >= n back-projection of bf16 parameters, two blocks per CU. A block of 4 waves
// holds a 256-row band of U in registers, 64 rows per wave (128 VGPRs), and walks up
// to kU2Tiles 32-row tiles of N: per tile its two planes are staged (32 KB, two
// buffers) and each wave multiplies them into a 32 x 64 block of C, so each fragment
// read serves twice the MFMAs of the 8-wave kernel and half the LDS reads are made.
// Two such blocks share a CU (2 x 80 KB of LDS). The parameter tile is loaded a
// tile ahead as there; to fit it beside U in 256 VGPRs, the stage's and the cells'
// addresses are recomputed per tile (from a lane index the compiler cannot hoist)
// instead of being held across the loop. Llama-7B list, bf16 parameters, side by
// side: 9.39-9.46 -> 9.15-9.27 ms, results bitwise the same. With fp32 parameters
// it gains nothing (12.33 -> 12.30 ms; the parameter stream bounds that pass), and
// those lists keep k_galore_back_ur.
constexpr int kU2N = 32;                     // rows of N per tile
constexpr int kU2Tiles = 2 * kUrTiles;       // tiles per item: the same 4096 rows of N
constexpr int kU2Dma = 2 * kU2N * (kGaWide / 8) / 256;  // 16-byte transfers per lane per tile: 8

__device__ __forceinline__ void u2_stage(const GDesc& d, int64_t n0, uint16_t* buf, int wave, int lane) {
    // instruction j: rows 2 jr, 2 jr + 1 of plane j / 16 (jr = j % 16), 32 chunks each
    __asm__ volatile("" : "+v"(lane));
#pragma unroll
    for (int i = 0; i < kU2Dma; ++i) {
        const int j = wave + 4 * i;                 // 0 .. 31
        const int plane = j >> 4, jr = j & 15;
        const int row = 2 * jr + (lane >> 5);       // 0 .. 31
        const int c = (lane & 31) ^ (row & 15);     // global chunk held at position lane & 31
        const int cc = min(c, d.r / 8 - 1);
        const int64_t grow = min(n0 + row, static_cast<int64_t>(d.D) - 1);
        const uint16_t* src = (plane ? d.nl : d.nh) + grow * d.r + cc * 8;
        __builtin_amdgcn_global_load_lds((const MEO_GLOBAL void*)src,
                                         (__attribute__((address_space(3))) void*)(buf + j * 512), 16, 0, 0);
    }
}

template <bool XB>
__global__ __launch_bounds__(256, 2) void k_galore_back_u2(GTable t, GaArgs a) {
    static_assert(kU2Dma == 8, "wait counts below");
    constexpr int kP = XB ? 4 : 8;  // 16-byte parameter loads (and stores) per lane per tile
    __shared__ __attribute__((aligned(16))) uint16_t nb0[2 * kU2N * 256];
    __shared__ __attribute__((aligned(16))) uint16_t nb1[2 * kU2N * 256];
    __shared__ __attribute__((aligned(16))) float exb[4 * 32 * 32];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of the XCD-dealt list
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nc = d.btj;
    const int band = it.y / nc, chunk = it.y % nc;
    const int64_t u0 = static_cast<int64_t>(band) * kGaWide;
    const int64_t nt0 = static_cast<int64_t>(chunk) * kU2Tiles;
    const int ntiles = static_cast<int>(min<int64_t>(kU2Tiles, (d.D + kU2N - 1) / kU2N - nt0));
    const int nks = d.r / 16;
    using PT = typename std::conditional<XB, uint16_t, float>::type;
    PT* const x = static_cast<PT*>(d.x);
    bfv8 uf[16][2];
#pragma unroll
    for (int ub = 0; ub < 2; ++ub) {
        const int64_t row = min(u0 + wave * 64 + ub * 32 + (lane & 31), static_cast<int64_t>(d.d) - 1);
#pragma unroll
        for (int ks = 0; ks < 16; ++ks) {
            const int k = min(ks, nks - 1) * 16 + 8 * (lane >> 5);
            uf[ks][ub] = __builtin_bit_cast(bfv8, *gld<u32x4>(d.u + row * d.r + k));
        }
    }
    MEO_WAIT_VM(0);
#pragma unroll
    for (int ks = 0; ks < 16; ++ks) __asm__ volatile("" : "+v"(uf[ks][0]), "+v"(uf[ks][1]));
    // W cells of the wave: the 32 tile rows x two 32-column blocks (ub); in block ub,
    // lane holds rows (lane >> 2) + 16 q (q < 2), columns 8 (lane & 3) .. + 7.
    auto cell = [&](int64_t n0, int ub, int q, int64_t& row, int64_t& col) {
        int ln = lane;
        __asm__ volatile("" : "+v"(ln));
        row = n0 + (ln >> 2) + 16 * q;
        col = u0 + wave * 64 + ub * 32 + 8 * (ln & 3);
    };
    u32x4 wp[2][2][2];  // [ub][q][16-byte half]
    auto load_w = [&](int64_t n0) {
        if (!d.wvec) return;
#pragma unroll
        for (int ub = 0; ub < 2; ++ub)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                int64_t row, col;
                cell(n0, ub, q, row, col);
                row = min(row, static_cast<int64_t>(d.m) - 1);
                col = min(col, static_cast<int64_t>(d.n) - 8);
                const PT* p = x + row * d.n + col;
                wp[ub][q][0] = *gld<u32x4>(p);
                if (!XB) wp[ub][q][1] = *gld<u32x4>(p + 4);
            }
    };
    f32x16 acc[2];
    auto multiply = [&](const uint16_t* buf) {
        // Fragment reads in asm blocks that wait for their own reads (the compiler
        // cannot tell which stage an LDS read hits). Two sub-steps per block; the low
        // plane sits 16 KB after the high one.
        static_assert(kU2N * 256 * 2 == 16384, "plane offset in the reads below");
        const uint32_t base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(buf)) + (lane & 31) * 512;
        const int sw = lane & 15;
#pragma unroll
        for (int ks = 0; ks < 16; ks += 2) {
            if (ks >= nks) break;
            int swv = sw;
            __asm__ volatile("" : "+v"(swv));
            const uint32_t a0 = base + static_cast<uint32_t>(((2 * ks + (lane >> 5)) ^ swv) << 4);
            const uint32_t a1 = base + static_cast<uint32_t>(((2 * ks + 2 + (lane >> 5)) ^ swv) << 4);
            u32x4 h0, l0, h1, l1;
            __asm__ volatile(
                "ds_read_b128 %0, %4\n\t"
                "ds_read_b128 %1, %4 offset:16384\n\t"
                "ds_read_b128 %2, %5\n\t"
                "ds_read_b128 %3, %5 offset:16384\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(h0), "=&v"(l0), "=&v"(h1), "=&v"(l1)
                : "v"(a0), "v"(a1));
            const bfv8 fh0 = __builtin_bit_cast(bfv8, h0), fl0 = __builtin_bit_cast(bfv8, l0);
            const bfv8 fh1 = __builtin_bit_cast(bfv8, h1), fl1 = __builtin_bit_cast(bfv8, l1);
#pragma unroll
            for (int ub = 0; ub < 2; ++ub) {
                acc[ub] = mfma32(fh0, uf[ks][ub], acc[ub]);
                acc[ub] = mfma32(fl0, uf[ks][ub], acc[ub]);
            }
#pragma unroll
            for (int ub = 0; ub < 2; ++ub) {
                acc[ub] = mfma32(fh1, uf[ks + 1][ub], acc[ub]);
                acc[ub] = mfma32(fl1, uf[ks + 1][ub], acc[ub]);
            }
        }
    };
    auto update = [&](int64_t n0, bool exact) {
        int lane = threadIdx.x & 63;
        __asm__ volatile("" : "+v"(lane));
        float* lw = exb + wave * (32 * 32);
#pragma unroll
        for (int ub = 0; ub < 2; ++ub) {
#pragma unroll
            for (int v = 0; v < 16; ++v) lw[ur_ex(acc_row(v, lane), acc_col(lane))] = acc[ub][v];
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                float cq[8];
                {
                    const int r = (lane >> 2) + 16 * q, c = 8 * (lane & 3);
                    const f32x4 c0 = *reinterpret_cast<const f32x4*>(lw + ur_ex(r, c));
                    const f32x4 c1 = *reinterpret_cast<const f32x4*>(lw + ur_ex(r, c + 4));
                    cq[0] = c0.x; cq[1] = c0.y; cq[2] = c0.z; cq[3] = c0.w;
                    cq[4] = c1.x; cq[5] = c1.y; cq[6] = c1.z; cq[7] = c1.w;
                }
                int64_t row, col;
                cell(n0, ub, q, row, col);
                float w[8];
                if (exact) {
                    PT* xp = x + row * d.n + col;
                    if (XB) {
                        bf16x8(wp[ub][q][0], w);
                    } else {
                        const u32x4 x0 = wp[ub][q][0], x1 = wp[ub][q][1];
                        w[0] = __uint_as_float(x0.x); w[1] = __uint_as_float(x0.y);
                        w[2] = __uint_as_float(x0.z); w[3] = __uint_as_float(x0.w);
                        w[4] = __uint_as_float(x1.x); w[5] = __uint_as_float(x1.y);
                        w[6] = __uint_as_float(x1.z); w[7] = __uint_as_float(x1.w);
                    }
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = a.decay * w[e] - a.coef * cq[e];
                    if (XB) {
                        *gst<u32x4>(xp) = pack_bf16x8(w);
                    } else {
                        *gst<f32x4>(xp) = f32x4{w[0], w[1], w[2], w[3]};
                        *gst<f32x4>(xp + 4) = f32x4{w[4], w[5], w[6], w[7]};
                    }
                } else {
                    if (row >= d.m || col >= d.n) continue;
                    PT* xp = x + row * d.n + col;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (col + e >= d.n) continue;
                        const float w0 = XB ? __uint_as_float(static_cast<uint32_t>(*gld<uint16_t>(reinterpret_cast<const uint16_t*>(xp) + e)) << 16)
                                            : *gld<float>(reinterpret_cast<const float*>(xp) + e);
                        const float w1 = a.decay * w0 - a.coef * cq[e];
                        if (XB) *gst<uint16_t>(reinterpret_cast<uint16_t*>(xp) + e) = static_cast<uint16_t>(bf16_bits(w1));
                        else *gst<float>(reinterpret_cast<float*>(xp) + e) = w1;
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (!exact) MEO_WAIT_VM(0);
    };
    auto zero = [&]() {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[b][v] = 0.0f;
    };
    const bool exact = d.wvec && (nt0 + ntiles) * kU2N <= d.D && u0 + kGaWide <= d.d;
    // The same pipeline and wait counts as the 8-wave kernel (8 stage transfers and kP
    // parameter loads or stores per lane per tile).
    const int last = ntiles - 1;
    u2_stage(d, nt0 * kU2N, nb0, wave, lane);
    u2_stage(d, (nt0 + min(1, last)) * kU2N, nb1, wave, lane);
    load_w(nt0 * kU2N);
    if (d.wvec) MEO_WAIT_VM(kP + 8);
    else MEO_WAIT_VM(8);
    for (int i = 0; i < ntiles; i += 2) {
        __builtin_amdgcn_s_barrier();
        zero();
        multiply(nb0);
        __builtin_amdgcn_s_barrier();
        update((nt0 + i) * kU2N, exact);
        if (i + 1 >= ntiles) break;
        u2_stage(d, (nt0 + min(i + 2, last)) * kU2N, nb0, wave, lane);
        load_w((nt0 + i + 1) * kU2N);
        if (exact) MEO_WAIT_VM(2 * kP + 8);
        else MEO_WAIT_VM(0);
        __builtin_amdgcn_s_barrier();
        zero();
        multiply(nb1);
        __builtin_amdgcn_s_barrier();
        update((nt0 + i + 1) * kU2N, exact);
        if (i + 2 >= ntiles) break;
        u2_stage(d, (nt0 + min(i + 3, last)) * kU2N, nb1, wave, lane);
        load_w((nt0 + i + 2) * kU2N);
        if (exact) MEO_WAIT_VM(2 * kP + 8);
        else MEO_WAIT_VM(0);
    }
    MEO_WAIT_VM(0);
}

void launch_galore_back(const GTable& t, int64_t n, const GaArgs& a, bool left, int mode, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kBackThreads);
    const bool direct = mode == kBackDirect;
    if (mode == kBackUr || mode == kBackUrBf16) {
        const bool xb = mode == kBackUrBf16;
        if (left && xb) hipLaunchKernelGGL((k_galore_back_ur<true, true>), grid, dim3(512), 0, s, t, a);
        else if (left) hipLaunchKernelGGL((k_galore_back_ur<true, false>), grid, dim3(512), 0, s, t, a);
        else if (xb) hipLaunchKernelGGL((k_galore_back_u2<true>), grid, dim3(256), 0, s, t, a);
        else hipLaunchKernelGGL((k_galore_back_ur<false, false>), grid, dim3(512), 0, s, t, a);
        return;
    }
    if (left) {
        if (direct) hipLaunchKernelGGL((k_galore_back<true, true>), grid, block, 0, s, t, a);
        else hipLaunchKernelGGL((k_galore_back<true, false>), grid, block, 0, s, t, a);
    } else {
        if (direct) hipLaunchKernelGGL((k_galore_back<false, true>), grid, block, 0, s, t, a);
        else hipLaunchKernelGGL((k_galore_back<false, false>), grid, block, 0, s, t, a);
    }
}

// ------------------------------------------------------------------ flat AdamW

// Tensors that are not 2-D: AdamW on every element (x, g fp32 or bf16; m, v fp32).
__global__ __launch_bounds__(kThreads) void k_galore_adamw(Table t, GaArgs a) {
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const bool vec = d.vec, bf = d.gbf16, xb = d.xbf16;
    const int64_t base = static_cast<int64_t>(it.y) * kFlatTile;
    float* m8 = static_cast<float*>(d.m);
    for (int k = 0; k < kFlatIters; ++k) {
        const int64_t i = base + (static_cast<int64_t>(k) * kThreads + threadIdx.x) * kVec;
        const int valid = clamp_valid(d.numel - i);
        if (valid == 0) break;
        float g[kVec], x[kVec], m[kVec], v[kVec];
        load_v8(d.g, i, valid, vec, bf, g);
        load_v8(d.x, i, valid, vec, xb, x);
        load_f8(m8 + i, valid, vec, m);
        load_f8(d.v + i, valid, vec, v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            m[e] = fmaf(a.beta1, m[e], a.omb1 * g[e]);
            v[e] = fmaf(a.beta2, v[e], a.omb2 * (g[e] * g[e]));
            const float n = (m[e] * a.inv_bc1) / (sqrtf(v[e] * a.inv_bc2) + a.eps);
            x[e] = a.decay * x[e] - a.coef * n;
        }
        store_f8(m8 + i, valid, vec, m);
        store_f8(d.v + i, valid, vec, v);
        store_v8(d.x, i, valid, vec, xb, x);
    }
}

void launch_galore_adamw(const Table& t, int64_t n, const GaArgs& a, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_galore_adamw, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, a);
}

}  // namespace meo
