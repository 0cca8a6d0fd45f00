// GaLore projector refresh: the leading r singular vectors of the gradient. The
// Colossal-AI distributed-optimizers page (section on GaLore's special
// configuration) redoes an SVD every update_proj_gap steps to refresh the
// orthogonal projection matrix; the ms-swift page (section on low-rank
// projection) keeps the leading singular directions. Only those r vectors are
// needed, so the refresh computes them by randomized subspace iteration with a
// Rayleigh-Ritz step (Halko, Martinsson and Tropp, "Finding structure with
// randomness", SIAM Review 2011, Algorithm 4.4 followed by the small SVD of
// Algorithm 5.1), with the gradient oriented as X (D x d) so that the wanted
// vectors span its rows' space:
//
//   Q^T (r x d) <- orthonormal rows of a Gaussian block (counter-based normals)
//   repeat kRfIters times:
//     Y^T = Q^T X^T   (r x D)          k_rf_gemm stage 0, bf16 MFMA, Q split in
//     Z^T = Y^T X     (r x d)          k_rf_gemm stage 1   two bf16 planes
//     Q^T <- orthonormal rows of Z^T   Cholesky-QR twice: k_rf_gram (fp64 Gram),
//                                      k_rf_chol (fp64 factor and its inverse),
//                                      k_rf_trmm (Q^T = L^-1 Z^T)
//   Y^T = Q^T X^T; S = Y^T Y (r x r, fp64) = W diag(sigma^2) W^T   k_rf_jacobi
//   U^T = (Q W)^T, columns by decreasing sigma                       k_rf_basis
//   each vector signed so that its largest-magnitude entry is positive, stored
//   in bf16 as U [d][r] and U^T [r][d]                               k_rf_store
//
// The result is the SVD's leading vectors up to the iteration's convergence,
// (sigma_{r+1} / sigma_r)^(2 kRfIters) for the subspace, and fp32 rounding.
#include "galore.h"

namespace meo {

typedef __bf16 bfv8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

namespace {

__device__ __forceinline__ f32x16 mfma32(const bfv8& a, const bfv8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float* rbuf(float* qa, float* qb, float* yt, int which) {
    return which == kRbQa ? qa : (which == kRbQb ? qb : yt);
}

// splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014): a counter-based 64-bit mix.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
    x += 0x9e3779b97f4a7c15ull;
    x = (x ^ (x >> 30)) * 0xbf58476d1ce4e5b9ull;
    x = (x ^ (x >> 27)) * 0x94d049bb133111ebull;
    return x ^ (x >> 31);
}

// A standard normal value for counter `key` (Box-Muller on two 24-bit uniforms).
__device__ __forceinline__ float normal_at(uint64_t key) {
    const uint64_t h = splitmix64(key);
    const float u1 = static_cast<float>((h >> 40) + 1) * (1.0f / 16777217.0f);  // (0, 1]
    const float u2 = static_cast<float>((h >> 16) & 0xffffffu) * (1.0f / 16777216.0f);
    return sqrtf(-2.0f * logf(u1)) * cospif(2.0f * u2);
}

__device__ __forceinline__ u32x4 ld_row8(const uint16_t* p, int64_t rows, int64_t cols, int64_t row, int64_t col,
                                         bool vec) {
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

__device__ __forceinline__ int acc_row(int v, int lane) { return 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3); }

constexpr int kRfBig = 1024;  // threads of the one-block-per-tensor kernels

// Block-wide sum / max of doubles over kRfBig threads (every thread gets the result).
__device__ double rf_sum_d(double v, double* lds) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = 0.0;
    for (int w = 0; w < kRfBig / 64; ++w) s += lds[w];
    return s;
}

__device__ double rf_max_d(double v, double* lds) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmax(v, __shfl_xor(v, o));
    __syncthreads();
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = v;
    __syncthreads();
    double s = lds[0];
    for (int w = 1; w < kRfBig / 64; ++w) s = fmax(s, lds[w]);
    return s;
}

}  // namespace

// ------------------------------------------------------------------ start block

// Start block: the stored projector's rows (U^T, zero before the first refresh)
// plus a Gaussian block scaled by 1e-6 / sqrt(d) (1e-6 of a unit vector's
// entries), one normal per element from the counter (tensor, index). The Gaussian
// keeps the block of full rank when there is no stored basis (the Cholesky-QR is
// scale-free) or it has lost rank; a stored basis close to the new one starts the
// iteration near its end, and the Rayleigh-Ritz matrix near diagonal: the
// perturbation's rotation inside the subspace, which the iteration does not
// remove, stays at 1e-6.
__global__ __launch_bounds__(kThreads) void k_rf_init(RTable t, int dst) {
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    float* out = rbuf(d.qa, d.qb, d.yt, dst);
    const int64_t total = static_cast<int64_t>(d.p) * d.d;
    const int64_t base = static_cast<int64_t>(it.y) * kThreads * kVec;
    const uint64_t key = static_cast<uint64_t>(d.seed) << 40;
    const float eps = 1e-6f / sqrtf(static_cast<float>(d.d));
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        const int64_t i = base + static_cast<int64_t>(e) * kThreads + threadIdx.x;
        if (i < total) {
            const float u = __uint_as_float(static_cast<uint32_t>(d.ut[i]) << 16);
            out[i] = fmaf(eps, normal_at(key + static_cast<uint64_t>(i)), u);
        }
    }
}

void launch_rf_init(const RTable& t, int64_t n, int dst, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_init, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, dst);
}

// ------------------------------------------------------------------ products with the gradient

// out[c][l] = sum_k in[c][k] B[l][k], c < p (fp32, split into two bf16 planes),
// B from the bf16 gradient G [m][n]: Trans = false reads B[l][k] = G[l][k] (G is
// [L][K]); Trans = true reads B[l][k] = G[k][l] (G is [K][L]), staged through LDS.
// Stage 0: L = D, K = d; stage 1: L = d, K = D. Tile: all p rows x 64 columns.
template <bool Trans>
__global__ __launch_bounds__(kThreads) void k_rf_gemm(RTable t, int stage, int src, int dst) {
    __shared__ __attribute__((aligned(16))) uint16_t ah[kRfMaxP * kRfPitch];
    __shared__ __attribute__((aligned(16))) uint16_t al[kRfMaxP * kRfPitch];
    __shared__ __attribute__((aligned(16))) uint16_t bs[kGaTile * kRfPitch];
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    const float* A = rbuf(d.qa, d.qb, d.yt, src);
    float* C = rbuf(d.qa, d.qb, d.yt, dst);
    const int64_t K = stage == 0 ? d.d : d.D;
    const int64_t L = stage == 0 ? d.D : d.d;
    const int64_t l0 = static_cast<int64_t>(it.y) * kGaTile;
    const int P = d.p;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const bool active = wave * 64 < P;
    const bool avec = (K & 3) == 0;
    f32x16 acc[2][2];
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[ib][jb][v] = 0.0f;

    // Staging: a thread's chunks of the next block are loaded into registers while
    // the current block is multiplied, then written to LDS.
    constexpr int kAPer = kRfMaxP * (kRfKb / 8) / kThreads;   // 8-float chunks of A
    constexpr int kBPer = kGaTile * (kRfKb / 8) / kThreads;   // 8-bf16 chunks of B
    f32x4 ra[kAPer][2];
    u32x4 rb[kBPer];
    auto fetch = [&](int64_t k0) {
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int row = c >> 2;
            const int64_t col = k0 + (c & 3) * 8;
            if (row < P && avec && col + 8 <= K) {
                ra[i][0] = *gld<f32x4>(A + row * K + col);
                ra[i][1] = *gld<f32x4>(A + row * K + col + 4);
            } else {
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = (row < P && col + e < K) ? A[row * K + col + e] : 0.0f;
                ra[i][0] = f32x4{v[0], v[1], v[2], v[3]};
                ra[i][1] = f32x4{v[4], v[5], v[6], v[7]};
            }
        }
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            if (!Trans) rb[i] = ld_row8(d.g, L, K, l0 + (c >> 2), k0 + (c & 3) * 8, d.gvec);
            else rb[i] = ld_row8(d.g, K, L, k0 + (c >> 3), l0 + (c & 7) * 8, d.gvec);
        }
    };
    auto put = [&]() {
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            const int row = c >> 2, kc = (c & 3) * 8;
            const float v[8] = {ra[i][0].x, ra[i][0].y, ra[i][0].z, ra[i][0].w,
                                ra[i][1].x, ra[i][1].y, ra[i][1].z, ra[i][1].w};
            float hi[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                hi[e] = round_bf16(v[e]);
                lo[e] = v[e] - hi[e];
            }
            *reinterpret_cast<u32x4*>(ah + row * kRfPitch + kc) = pack_bf16x8(hi);
            *reinterpret_cast<u32x4*>(al + row * kRfPitch + kc) = pack_bf16x8(lo);
        }
#pragma unroll
        for (int i = 0; i < kBPer; ++i) {
            const int c = threadIdx.x + i * kThreads;
            if (!Trans) {
                *reinterpret_cast<u32x4*>(bs + (c >> 2) * kRfPitch + (c & 3) * 8) = rb[i];
            } else {
                const int k = c >> 3, lc = (c & 7) * 8;
                const uint32_t w[4] = {rb[i].x, rb[i].y, rb[i].z, rb[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    bs[(lc + 2 * e) * kRfPitch + k] = static_cast<uint16_t>(w[e] & 0xffffu);
                    bs[(lc + 2 * e + 1) * kRfPitch + k] = static_cast<uint16_t>(w[e] >> 16);
                }
            }
        }
    };
    fetch(0);
    for (int64_t k0 = 0; k0 < K; k0 += kRfKb) {
        put();
        __syncthreads();
        if (k0 + kRfKb < K) fetch(k0 + kRfKb);
        if (active) {
#pragma unroll
            for (int ks = 0; ks < kRfKb; ks += 16) {
                const int kk = ks + 8 * (lane >> 5);
                bfv8 fh[2], fl[2], fb[2];
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const int r = wave * 64 + b * 32 + (lane & 31);
                    fh[b] = *reinterpret_cast<const bfv8*>(ah + r * kRfPitch + kk);
                    fl[b] = *reinterpret_cast<const bfv8*>(al + r * kRfPitch + kk);
                    fb[b] = *reinterpret_cast<const bfv8*>(bs + (b * 32 + (lane & 31)) * kRfPitch + kk);
                }
#pragma unroll
                for (int ib = 0; ib < 2; ++ib)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) {
                        acc[ib][jb] = mfma32(fh[ib], fb[jb], acc[ib][jb]);
                        acc[ib][jb] = mfma32(fl[ib], fb[jb], acc[ib][jb]);
                    }
            }
        }
        __syncthreads();
    }
    if (!active) return;
#pragma unroll
    for (int ib = 0; ib < 2; ++ib)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int64_t l = l0 + jb * 32 + (lane & 31);
            if (l >= L) continue;
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wave * 64 + ib * 32 + acc_row(v, lane);
                if (row < P) C[row * L + l] = acc[ib][jb][v];
            }
        }
}

void launch_rf_gemm(const RTable& t, int64_t n, int stage, int src, int dst, bool trans, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (trans) hipLaunchKernelGGL(k_rf_gemm<true>, grid, block, 0, s, t, stage, src, dst);
    else hipLaunchKernelGGL(k_rf_gemm<false>, grid, block, 0, s, t, stage, src, dst);
}

// ------------------------------------------------------------------ Gram matrix (fp64)

// S[a][b] = sum_k A[a][k] A[b][k] over the p rows of `src` (length d, or D when
// over_long): products of fp32 values are exact in fp64 and summed in fp64.
__global__ __launch_bounds__(kThreads) void k_rf_gram(RTable t, int src, int over_long) {
    __shared__ float sa[64][33];
    __shared__ float sb[64][33];
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    const float* A = rbuf(d.qa, d.qb, d.yt, src);
    const int64_t K = over_long ? d.D : d.d;
    const int P = d.p;
    const int tp = (P + 63) / 64;
    const int a0 = (it.y / tp) * 64, b0 = (it.y % tp) * 64;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    for (int64_t k0 = 0; k0 < K; k0 += 32) {
        for (int c = threadIdx.x; c < 64 * 32; c += kThreads) {
            const int r = c >> 5, k = c & 31;
            const bool kin = k0 + k < K;
            sa[r][k] = (a0 + r < P && kin) ? A[(a0 + r) * K + k0 + k] : 0.0f;
            sb[r][k] = (b0 + r < P && kin) ? A[(b0 + r) * K + k0 + k] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < 32; ++k) {
            double av[4], bv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                av[i] = static_cast<double>(sa[ty * 4 + i][k]);
                bv[i] = static_cast<double>(sb[tx * 4 + i][k]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int a = a0 + ty * 4 + i, b = b0 + tx * 4 + j;
            if (a < P && b < P) d.s[a * P + b] = acc[i][j];
        }
}

void launch_rf_gram(const RTable& t, int64_t n, int src, bool over_long, hipStream_t s) {
    if (n > 0)
        hipLaunchKernelGGL(k_rf_gram, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, src,
                           over_long ? 1 : 0);
}

// ------------------------------------------------------------------ Cholesky factor and its inverse

// One block per tensor: S <- L (lower, in place) with S + 1e-13 max(diag S) I =
// L L^T, then W <- L^-1 (lower). The shift keeps a numerically rank-deficient
// block finite; a pivot that is not positive is replaced by 1. The inverse is
// taken 16 columns at a time, one wave per column, the column kept in LDS and
// each row's sum split over the wave's lanes.
__global__ __launch_bounds__(kRfBig) void k_rf_chol(RTable t) {
    __shared__ double red[kRfBig / 64];
    __shared__ double inv;
    __shared__ double col[kRfBig / 64][kRfMaxP];
    const RDesc d = t.desc[t.items[blockIdx.x].x];
    double* S = d.s;
    double* W = d.w;
    const int P = d.p;
    const int tid = threadIdx.x;
    double mx = 0.0;
    for (int i = tid; i < P; i += kRfBig) mx = fmax(mx, S[i * P + i]);
    mx = rf_max_d(mx, red);
    const double shift = 1e-13 * mx;
    for (int i = tid; i < P; i += kRfBig) S[i * P + i] += shift;
    __syncthreads();
    for (int k = 0; k < P; ++k) {
        if (tid == 0) {
            const double piv = S[k * P + k];
            const double lkk = (piv > 0.0 && piv < INFINITY) ? sqrt(piv) : 1.0;
            S[k * P + k] = lkk;
            inv = 1.0 / lkk;
        }
        __syncthreads();
        for (int i = k + 1 + tid; i < P; i += kRfBig) S[i * P + k] *= inv;
        __syncthreads();
        const int j = k + 1 + (tid & (kRfMaxP - 1));
        if (j < P) {
            const double sjk = S[j * P + k];
            for (int i = k + 1 + (tid >> 8); i < P; i += kRfBig / kRfMaxP)
                if (j <= i) S[i * P + j] = fma(-S[i * P + k], sjk, S[i * P + j]);
        }
        __syncthreads();
    }
    // W = L^-1: column j solves L w = e_j; w_i = -(sum_{j<=k<i} L_ik w_k) / L_ii.
    const int lane = tid & 63, wv = tid >> 6;
    double* cw = col[wv];
    for (int j = wv; j < P; j += kRfBig / 64) {
        for (int i = lane; i < P; i += 64) cw[i] = 0.0;
        if (lane == 0) cw[j] = 1.0 / S[j * P + j];
        for (int i = j + 1; i < P; ++i) {
            double acc = 0.0;
            for (int k = j + lane; k < i; k += 64) acc = fma(S[i * P + k], cw[k], acc);
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
            if (lane == 0) cw[i] = -acc / S[i * P + i];
            __builtin_amdgcn_wave_barrier();  // lane 0's write precedes the next row's reads
        }
        for (int i = lane; i < P; i += 64) W[i * P + j] = cw[i];
    }
}

void launch_rf_chol(const RTable& t, int64_t n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_chol, dim3(static_cast<uint32_t>(n)), dim3(kRfBig), 0, s, t);
}

// out[a][j] = sum_b M[a][b] src[b][j] over the p x d block `src`, one 64 x 64 tile
// of `out` per block: M's 64 x 32 and src's 32 x 64 slices staged in LDS, a 4 x 4
// fp64 sub-tile per thread (columns contiguous for the stores).
//   Tri:   M = W (lower triangular, the inverse factor), a < p rows; slices of b
//          beyond the tile's last row are zero and skipped.
//   Basis: M[c][b] = W[b][o_c] (eigenvector o_c, o sorting the eigenvalues on S's
//          diagonal in decreasing order, ties by index), c < r rows.
template <bool Basis>
__device__ __forceinline__ void rf_small_product(const RDesc& d, const float* src, float* out, int tile) {
    __shared__ double ms[64][33];
    __shared__ float zs[32][68];
    __shared__ int ord[kRfMaxP];
    const int P = d.p;
    const int rows = Basis ? d.r : P;
    const int tjn = (d.d + 63) / 64;
    const int a0 = (tile / tjn) * 64;
    const int64_t j0 = static_cast<int64_t>(tile % tjn) * 64;
    const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
    if (Basis) {
        for (int i = tid; i < P; i += kThreads) {
            const double li = d.s[i * P + i];
            int rank = 0;
            for (int k = 0; k < P; ++k) {
                const double lk = d.s[k * P + k];
                rank += (lk > li || (lk == li && k < i)) ? 1 : 0;
            }
            ord[rank] = i;
        }
    }
    double acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
    const int bend = Basis ? P : (a0 + 64 < P ? a0 + 64 : P);
    for (int b0 = 0; b0 < bend; b0 += 32) {
        __syncthreads();  // also orders `ord` before its first use
        for (int c = tid; c < 64 * 32; c += kThreads) {
            const int i = c >> 5, k = c & 31;
            const int a = a0 + i, b = b0 + k;
            double v = 0.0;
            if (a < rows && b < P) v = Basis ? d.w[b * P + ord[a]] : d.w[a * P + b];
            ms[i][k] = v;
        }
        for (int c = tid; c < 32 * 64; c += kThreads) {
            const int k = c >> 6, jj = c & 63;
            const int b = b0 + k;
            zs[k][jj] = (b < P && j0 + jj < d.d) ? src[b * static_cast<int64_t>(d.d) + j0 + jj] : 0.0f;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < 32; ++k) {
            double mv[4], zv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                mv[i] = ms[ty * 4 + i][k];
                zv[i] = static_cast<double>(zs[k][tx * 4 + i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fma(mv[i], zv[j], acc[i][j]);
        }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int a = a0 + ty * 4 + i;
        if (a >= rows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t jj = j0 + tx * 4 + j;
            if (jj < d.d) out[a * static_cast<int64_t>(d.d) + jj] = static_cast<float>(acc[i][j]);
        }
    }
}

// Q^T = L^-1 Z^T (the triangular factor's inverse in W).
__global__ __launch_bounds__(kThreads) void k_rf_trmm(RTable t, int src, int dst) {
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    rf_small_product<false>(d, rbuf(d.qa, d.qb, d.yt, src), rbuf(d.qa, d.qb, d.yt, dst), it.y);
}

void launch_rf_trmm(const RTable& t, int64_t n, int src, int dst, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_trmm, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, src, dst);
}

// ------------------------------------------------------------------ symmetric eigenproblem (fp64)

// One block per tensor: cyclic Jacobi with the round-robin ordering, so each round
// applies p/2 disjoint rotations at once: S <- J^T S J, W <- W J, with J's column
// a holding c_a at a and t_a at its partner (t = -s for the first of a pair, +s
// for the second). Rotation angles as in the classical method (Rutishauser's
// formulation: tan of the angle from theta = (S_jj - S_ii) / (2 S_ij)). Stops when
// the off-diagonal norm is below 1e-9 of the whole (an eigenvector then moves by
// about 1e-9 over its gap relative to the largest eigenvalue, 1e-5 for gaps of
// 1e-4; the stored basis is rounded to bf16, 4e-3), or after 16 sweeps. On exit
// S holds the eigenvalues on its diagonal and W the eigenvectors as columns.
__global__ __launch_bounds__(kRfBig) void k_rf_jacobi(RTable t) {
    __shared__ double cc[kRfMaxP + 1], tt[kRfMaxP + 1];
    __shared__ int qq[kRfMaxP + 1];
    __shared__ double red[kRfBig / 64];
    const RDesc d = t.desc[t.items[blockIdx.x].x];
    const int P = d.p;
    const int Pe = P + (P & 1);  // an odd size gets a dummy index P
    const int tid = threadIdx.x;
    const int b = tid & (kRfMaxP - 1), a0 = tid >> 8;  // column, first row of this thread
    constexpr int kRowStep = kRfBig / kRfMaxP;
    double* S = d.s;
    double* W = d.w;
    double* S2 = d.s2;
    double* W2 = d.w2;
    if (b < P)
        for (int a = a0; a < P; a += kRowStep) W[a * P + b] = a == b ? 1.0 : 0.0;
    __syncthreads();
    for (int sweep = 0; sweep < 16; ++sweep) {
        double off = 0.0, tot = 0.0;
        if (b < P)
            for (int a = a0; a < P; a += kRowStep) {
                const double v = S[a * P + b] * S[a * P + b];
                tot += v;
                if (a != b) off += v;
            }
        off = rf_sum_d(off, red);
        tot = rf_sum_d(tot, red);
        if (!(off > 1e-18 * tot)) break;  // uniform: every thread holds the same sums
        for (int round = 0; round < Pe - 1; ++round) {
            // pairs of the circle method: 0 with 1 + round, and the rest mirrored
            if (tid < Pe / 2) {
                const int k = tid;
                int i, j;
                if (k == 0) {
                    i = 0;
                    j = 1 + round;
                } else {
                    i = 1 + (round + k) % (Pe - 1);
                    j = 1 + (round + Pe - 1 - k) % (Pe - 1);
                }
                if (i > j) { const int x = i; i = j; j = x; }
                double c = 1.0, s = 0.0;
                if (j < P) {
                    const double sij = S[i * P + j];
                    if (sij != 0.0) {
                        const double theta = (S[j * P + j] - S[i * P + i]) / (2.0 * sij);
                        const double tn = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(fma(theta, theta, 1.0)));
                        c = 1.0 / sqrt(fma(tn, tn, 1.0));
                        s = tn * c;
                    }
                }
                cc[i] = c; tt[i] = -s; qq[i] = j;
                cc[j] = c; tt[j] = s; qq[j] = i;
            }
            __syncthreads();
            if (b < P) {
                const int qb = qq[b];
                const double cb = cc[b], tb = tt[b];
                for (int a = a0; a < P; a += kRowStep) {
                    const int qa = qq[a];
                    const double ca = cc[a], ta = tt[a];
                    double v = ca * cb * S[a * P + b];
                    if (qb < P) v = fma(ca * tb, S[a * P + qb], v);
                    if (qa < P) v = fma(ta * cb, S[qa * P + b], v);
                    if (qa < P && qb < P) v = fma(ta * tb, S[qa * P + qb], v);
                    S2[a * P + b] = v;
                    double w = cb * W[a * P + b];
                    if (qb < P) w = fma(tb, W[a * P + qb], w);
                    W2[a * P + b] = w;
                }
            }
            __syncthreads();
            double* x = S; S = S2; S2 = x;
            x = W; W = W2; W2 = x;
        }
    }
    if (S != d.s && b < P) {  // leave the result in s and w
        for (int a = a0; a < P; a += kRowStep) {
            d.s[a * P + b] = S[a * P + b];
            d.w[a * P + b] = W[a * P + b];
        }
    }
}

void launch_rf_jacobi(const RTable& t, int64_t n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_jacobi, dim3(static_cast<uint32_t>(n)), dim3(kRfBig), 0, s, t);
}

// ------------------------------------------------------------------ basis and storage

// U^T[c][j] = sum_b W[b][o_c] Q^T[b][j] for c < r, where o sorts the eigenvalues
// (diagonal of S) in decreasing order (ties by index); written as fp32 [r][d]
// into the yt buffer.
__global__ __launch_bounds__(kThreads) void k_rf_basis(RTable t, int src) {
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    rf_small_product<true>(d, rbuf(d.qa, d.qb, d.yt, src), d.yt, it.y);
}

void launch_rf_basis(const RTable& t, int64_t n, int src, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_basis, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, src);
}

// One block per (tensor, vector c): the sign that makes the largest-magnitude entry
// (first on a tie) positive, then U^T[c][:] and U[:][c] in bf16.
__global__ __launch_bounds__(kThreads) void k_rf_store(RTable t) {
    __shared__ float bv[kWaves];
    __shared__ int bi[kWaves];
    __shared__ float sign;
    const int2 it = t.items[blockIdx.x];
    const RDesc d = t.desc[it.x];
    const int c = it.y;
    const float* row = d.yt + c * static_cast<int64_t>(d.d);
    float best = -1.0f;
    int bidx = 0x7fffffff;
    for (int j = threadIdx.x; j < d.d; j += kThreads) {
        const float a = fabsf(row[j]);
        if (a > best) { best = a; bidx = j; }  // j increases: first index on a tie
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        const float ob = __shfl_xor(best, o);
        const int oi = __shfl_xor(bidx, o);
        if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
    }
    if ((threadIdx.x & 63) == 0) { bv[threadIdx.x >> 6] = best; bi[threadIdx.x >> 6] = bidx; }
    __syncthreads();
    if (threadIdx.x == 0) {
        float b = bv[0];
        int i = bi[0];
        for (int w = 1; w < kWaves; ++w)
            if (bv[w] > b || (bv[w] == b && bi[w] < i)) { b = bv[w]; i = bi[w]; }
        sign = (i < d.d && row[i] < 0.0f) ? -1.0f : 1.0f;
    }
    __syncthreads();
    const float sg = sign;
    for (int j = threadIdx.x; j < d.d; j += kThreads) {
        const uint16_t v = static_cast<uint16_t>(bf16_bits(sg * row[j]));
        d.ut[c * static_cast<int64_t>(d.d) + j] = v;
        d.u[static_cast<int64_t>(j) * d.r + c] = v;
    }
}

void launch_rf_store(const RTable& t, int64_t n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rf_store, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t);
}

}  // namespace meo
