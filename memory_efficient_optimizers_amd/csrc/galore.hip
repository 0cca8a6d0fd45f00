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
//   k_galore_project  R = X U with X = G (m >= n) or G^T (m < n), bf16 MFMA with
//                     fp32 accumulation, one 64-row tile of R per block and the
//                     whole contraction in the block (no split partials); the
//                     epilogue runs AdamW on the tile: moments updated in place,
//                     direction N = m_hat / (sqrt(v_hat) + eps) written as two
//                     bf16 planes (high part and the remainder) so that the back
//                     projection keeps ~16 significant bits of N on bf16 MFMA.
//   k_galore_back     W <- W (1 - lr wd) - lr scale (N U^T or U N^T): two bf16
//                     MFMAs per fragment (high and low plane), the parameter tile
//                     read and written once.
//
// The projector is kept in bf16 (the gradient's type) both as U [d][r] and as
// U^T [r][d], so every operand is read with the contraction index contiguous.
// The only transposed read is G in the m < n projection, which is staged through
// LDS. Non-projected tensors take a flat AdamW kernel (k_galore_adamw).
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
template <int NROWS>
struct RowStage {
    static constexpr int kPer = NROWS * (kGaKb / 8) / kThreads;
    u32x4 v[kPer];
    __device__ __forceinline__ void load(const uint16_t* p, int64_t rows, int64_t cols, int64_t r0, int64_t k0,
                                         bool vec) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            v[i] = ld_row8(p, rows, cols, r0 + (c >> 3), k0 + (c & 7) * 8, vec);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            st_lds8(lds + (c >> 3) * kGaPitch + (c & 7) * 8, v[i]);
        }
    }
};

// The transposed tile A[i][k] = G[k0 + k][i0 + i] (i < kGaTile, k < kGaKb) of the
// row-major gradient G [K][D]: loaded along G's rows, scattered into LDS.
struct TransStage {
    static constexpr int kPer = kGaKb * (kGaTile / 8) / kThreads;
    u32x4 v[kPer];
    __device__ __forceinline__ void load(const uint16_t* g, int64_t K, int64_t D, int64_t i0, int64_t k0, bool vec) {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            v[i] = ld_row8(g, K, D, k0 + (c >> 3), i0 + (c & 7) * 8, vec);
        }
    }
    __device__ __forceinline__ void store(uint16_t* lds) const {
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int k = c >> 3, ic = (c & 7) * 8;
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

// ------------------------------------------------------------------ projection + AdamW

template <bool Left>
__global__ __launch_bounds__(kThreads) void k_galore_project(GTable t, GaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sa[kGaTile * kGaPitch];
    __shared__ __attribute__((aligned(16))) uint16_t sb[kGaWide * kGaPitch];
    const int2 it = t.items[blockIdx.x];
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t i0 = static_cast<int64_t>(it.y) * kGaTile;
    const bool vec = d.vec, active = wave * 64 < d.r;
    f32x16 acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.0f;

    typename std::conditional<Left, TransStage, RowStage<kGaTile>>::type pa;
    RowStage<kGaWide> pb;
    auto fetch = [&](int64_t k0) {
        if constexpr (Left) pa.load(d.g, d.d, d.D, i0, k0, vec);
        else pa.load(d.g, d.D, d.d, i0, k0, vec);
        pb.load(d.ut, d.r, d.d, 0, k0, vec);
    };
    fetch(0);
    for (int64_t k0 = 0; k0 < d.d; k0 += kGaKb) {
        pa.store(sa);
        pb.store(sb);
        __syncthreads();
        if (k0 + kGaKb < d.d) fetch(k0 + kGaKb);
        if (active) {
#pragma unroll
            for (int ks = 0; ks < kGaKb; ks += 16) {
                const int kk = ks + 8 * (lane >> 5);
                bfv8 fa[2], fb[2];
#pragma unroll
                for (int ib = 0; ib < 2; ++ib) fa[ib] = ld_frag(sa + (ib * 32 + (lane & 31)) * kGaPitch + kk);
#pragma unroll
                for (int jb = 0; jb < 2; ++jb)
                    fb[jb] = ld_frag(sb + (wave * 64 + jb * 32 + (lane & 31)) * kGaPitch + kk);
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) acc[ib][jb] = mfma32(fa[ib], fb[jb], acc[ib][jb]);
            }
        }
        __syncthreads();
    }
    if (!active) return;
    // AdamW on the tile of R: lanes 0..31 of an accumulator register hold 32
    // consecutive columns of one row. The moments of a 32x32 block are loaded
    // together, then updated and stored.
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int col = wave * 64 + jb * 32 + acc_col(lane);
            const bool cok = col < d.r;
            float m0[16], v0[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = i0 + ib * 32 + acc_row(v, lane);
                const bool ok = cok && row < d.D;
                const int64_t idx = row * d.r + col;
                m0[v] = ok ? *gld<float>(d.em + idx) : 0.0f;
                v0[v] = ok ? *gld<float>(d.ev + idx) : 0.0f;
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = i0 + ib * 32 + acc_row(v, lane);
                if (!cok || row >= d.D) continue;
                const int64_t idx = row * d.r + col;
                const float rv = acc[ib][jb][v];
                const float m = fmaf(a.beta1, m0[v], a.omb1 * rv);
                const float vv = fmaf(a.beta2, v0[v], a.omb2 * (rv * rv));
                *gst<float>(d.em + idx) = m;
                *gst<float>(d.ev + idx) = vv;
                const float n = (m * a.inv_bc1) / (sqrtf(vv * a.inv_bc2) + a.eps);
                const __bf16 hi = static_cast<__bf16>(n);
                const __bf16 lo = static_cast<__bf16>(n - static_cast<float>(hi));
                *gst<uint16_t>(d.nh + idx) = __builtin_bit_cast(uint16_t, hi);
                *gst<uint16_t>(d.nl + idx) = __builtin_bit_cast(uint16_t, lo);
            }
        }
}

void launch_galore_project(const GTable& t, int64_t n, const GaArgs& a, bool left, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (left) hipLaunchKernelGGL(k_galore_project<true>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_galore_project<false>, grid, block, 0, s, t, a);
}

// ------------------------------------------------------------------ back-projection + update

// m >= n: tile 64 rows x 256 columns of W; C = Nh U^T + Nl U^T, waves along columns.
// m <  n: tile 256 rows x 64 columns; C = U Nh^T + U Nl^T, waves along rows.
template <bool Left>
__global__ __launch_bounds__(kThreads) void k_galore_back(GTable t, GaArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t sh[kGaTile * kGaPitch];   // N, high plane
    __shared__ __attribute__((aligned(16))) uint16_t sl[kGaTile * kGaPitch];   // N, low plane
    __shared__ __attribute__((aligned(16))) uint16_t su[kGaWide * kGaPitch];   // U rows
    const int2 it = t.items[blockIdx.x];
    const GDesc d = t.desc[it.x];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int ti = it.y / d.btj, tj = it.y % d.btj;
    // Tile origin in W; the 64-wide side indexes N's rows, the 256-wide side U's rows.
    const int64_t r0 = Left ? static_cast<int64_t>(ti) * kGaWide : static_cast<int64_t>(ti) * kGaTile;
    const int64_t c0 = Left ? static_cast<int64_t>(tj) * kGaTile : static_cast<int64_t>(tj) * kGaWide;
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

    RowStage<kGaTile> ph, pl;
    RowStage<kGaWide> pu;
    auto fetch = [&](int k0) {
        ph.load(d.nh, d.D, d.r, n0, k0, vec);
        pl.load(d.nl, d.D, d.r, n0, k0, vec);
        pu.load(d.u, d.d, d.r, u0, k0, vec);
    };
    fetch(0);
    for (int k0 = 0; k0 < d.r; k0 += kGaKb) {
        ph.store(sh);
        pl.store(sl);
        pu.store(su);
        __syncthreads();
        if (k0 + kGaKb < d.r) fetch(k0 + kGaKb);
#pragma unroll
        for (int ks = 0; ks < kGaKb; ks += 16) {
            const int kk = ks + 8 * (lane >> 5);
            bfv8 fu[2], fh[2], fl[2];
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                fu[b] = ld_frag(su + (wave * 64 + b * 32 + (lane & 31)) * kGaPitch + kk);
                fh[b] = ld_frag(sh + (b * 32 + (lane & 31)) * kGaPitch + kk);
                fl[b] = ld_frag(sl + (b * 32 + (lane & 31)) * kGaPitch + kk);
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
        __syncthreads();
    }
    // W <- decay W - coef C; lanes 0..31 of a register hold 32 consecutive
    // columns. The parameters of a 32x32 block are loaded together, then stored.
    const int64_t wr0 = Left ? r0 + wave * 64 : r0;
    const int64_t wc0 = Left ? c0 : c0 + wave * 64;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int64_t col = wc0 + jb * 32 + acc_col(lane);
            const bool cok = col < d.n;
            float w[16];
            if (d.xbf16) {
                const uint16_t* xp = static_cast<const uint16_t*>(d.x);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = wr0 + ib * 32 + acc_row(v, lane);
                    w[v] = (cok && row < d.m) ? __uint_as_float(static_cast<uint32_t>(*gld<uint16_t>(xp + row * d.n + col)) << 16)
                                              : 0.0f;
                }
            } else {
                const float* xp = static_cast<const float*>(d.x);
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    const int64_t row = wr0 + ib * 32 + acc_row(v, lane);
                    w[v] = (cok && row < d.m) ? *gld<float>(xp + row * d.n + col) : 0.0f;
                }
            }
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int64_t row = wr0 + ib * 32 + acc_row(v, lane);
                if (!cok || row >= d.m) continue;
                const float nw = a.decay * w[v] - a.coef * acc[ib][jb][v];
                if (d.xbf16) *gst<uint16_t>(static_cast<uint16_t*>(d.x) + row * d.n + col) = static_cast<uint16_t>(bf16_bits(nw));
                else *gst<float>(static_cast<float*>(d.x) + row * d.n + col) = nw;
            }
        }
}

void launch_galore_back(const GTable& t, int64_t n, const GaArgs& a, bool left, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (left) hipLaunchKernelGGL(k_galore_back<true>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_galore_back<false>, grid, block, 0, s, t, a);
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
