// Passes shared by Adafactor and CAME (and the scalar pass shared with LAMB).
//
//   k_stats     read G once: per-tile row sums and column sums of Q = G^2 + eps1
//               (factored tensors), or the full 1-D statistic V <- beta V +
//               (1-beta) Q with per-tile sums of U^2 = G^2 / V (and x^2).
//   k_finalize  fold the tile partials into the row and column statistics:
//               s <- beta s + (1 - beta) mean, in fp64, fixed order; per-chunk sums
//               of the new row statistic for its mean.
//   k_rms       read G (and X) again: per-tile sums of U^2 with
//               U = G rsqrt(R_i / mean(R)) rsqrt(C_j) rebuilt on the fly (the
//               [H, W] estimate is never stored), and of x^2.
//   k_scalars   one block per tensor: RMS(U), RMS(X), the clip divisor and the
//               per-matrix coefficients used by the apply passes.
//
// The factored statistics follow the "four optimizers" table of the Colossal-AI
// distributed-optimizers page (second moment approximated by row * col) and its
// section "Step 3" (row statistic [H], column statistic [W], full statistic for
// 1-D tensors); RMS clipping and the step-size rules follow the note after its
// "Step 5".
#include "internal.h"

namespace meo {

// ----------------------------------------------------------------------------- k_stats

__device__ void stats_factored(const TDesc& d, int64_t lt, float* __restrict__ ws, const StatsArgs& a,
                               float* lds) {
    const TileRC p = tile_rc(d, lt);
    const int lane = threadIdx.x & 63;
    const bool vec = d.vec, bf = d.gbf16;
    const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
    float* rowpart = ws + d.rowpart + (static_cast<int64_t>(p.b) * d.tc + p.ct) * d.H;
    float cs[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) cs[e] = 0.0f;

    for (int i0 = 0; i0 < p.nrows; i0 += 8) {
        float g[8][kVec];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i0 + i < p.nrows)
                load_g8<true>(d.g, mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, bf, g[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i0 + i < p.nrows) {
                float rs = 0.0f;
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    const float q = e < p.valid ? fmaf(g[i][e], g[i][e], a.eps1) : 0.0f;
                    cs[e] += q;
                    rs += q;
                }
                rs = wave_sum(rs);
                if (lane == 0) stf(rowpart + p.row0 + i0 + i, rs);
            }
        }
    }
    write_colpart(d, ws, p, cs, lds);
}

__device__ void stats_flat(const TDesc& d, int64_t lt, float* __restrict__ ws, const StatsArgs& a,
                           float* lds) {
    const bool vec = d.vec, bf = d.gbf16;
    const float beta = a.beta, omb = a.omb;
    const int64_t base = lt * kFlatTile;
    float su[kVec], sx[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) { su[e] = 0.0f; sx[e] = 0.0f; }
    for (int it = 0; it < kFlatIters; ++it) {
        const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
        const int valid = clamp_valid(d.numel - i);
        if (valid == 0) break;
        float g[kVec], v[kVec] = {};
        load_g8(d.g, i, valid, vec, bf, g);
        if (beta != 0.0f) load_f8(d.v + i, valid, vec, v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const float q = fmaf(g[e], g[e], a.eps1);
            v[e] = beta != 0.0f ? fmaf(beta, v[e], omb * q) : q;
            const float u = e < valid ? g[e] * rsqrtf(v[e]) : 0.0f;
            su[e] = fmaf(u, u, su[e]);
        }
        store_f8(d.v + i, valid, vec, v);
        if (a.need_x) {
            float x[kVec];
            load_f8(d.x + i, valid, vec, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
        }
    }
    float tu = sum8(su), tx = sum8(sx);
    block_sum2(tu, tx, lds);
    if (threadIdx.x == 0) {
        float* tp = ws + d.tilepart + 2 * lt;
        stf(tp, tu);
        stf(tp + 1, tx);
    }
}

__global__ __launch_bounds__(kThreads) void k_stats(Table t, StatsArgs a) {
    __shared__ __align__(16) float lds[kWaves * kTileCols];
    const int64_t tile = blockIdx.x;
    const int k = tensor_of(t.tile_tensor, tile);
    const TDesc d = t.desc[k];
    const int64_t lt = tile - d.tile0;
    if (d.factored) stats_factored(d, lt, t.ws, a, lds);
    else stats_flat(d, lt, t.ws, a, lds);
}

void launch_stats(const Table& t, int64_t tiles, const StatsArgs& a, hipStream_t s) {
    if (tiles > 0) hipLaunchKernelGGL(k_stats, dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0, s, t, a);
}

// ----------------------------------------------------------------------------- k_finalize

// Items of a factored tensor, per matrix b: nrc row chunks then ncc column chunks.
__global__ __launch_bounds__(kThreads) void k_finalize(Table t, FinArgs a) {
    __shared__ double lds[kWaves];
    const int64_t item = blockIdx.x;
    const int k = tensor_of(t.fin_tensor, item);
    const TDesc d = t.desc[k];
    const int64_t li = item - d.fin0;
    const int per = d.nrc + d.ncc;
    const int b = static_cast<int>(li / per);
    const int j = static_cast<int>(li - static_cast<int64_t>(b) * per);
    float* ws = t.ws;
    float* rs = a.which ? d.rr : d.r;
    float* cs = a.which ? d.rc : d.c;
    const double beta = a.beta, omb = 1.0 - a.beta;
    if (j < d.nrc) {
        const int row = j * kFinChunk + threadIdx.x;
        double rnew = 0.0;
        if (row < d.H) {
            const float* rp = ws + d.rowpart + static_cast<int64_t>(b) * d.tc * d.H + row;
            double s = 0.0;
            for (int ct = 0; ct < d.tc; ++ct) s += static_cast<double>(ldf(rp + static_cast<int64_t>(ct) * d.H));
            float* dst = rs + static_cast<int64_t>(b) * d.H + row;
            const double mean = s / static_cast<double>(d.W);
            rnew = beta != 0.0 ? beta * static_cast<double>(ldf(dst)) + omb * mean : mean;
            const float r32 = static_cast<float>(rnew);
            stf(dst, r32);
            rnew = static_cast<double>(r32);  // the mean is taken over the stored values
        }
        const double tot = block_sum_d(rnew, lds);
        if (threadIdx.x == 0) stf(ws + d.sumr + static_cast<int64_t>(b) * d.nrc + j, static_cast<float>(tot));
    } else {
        const int col = (j - d.nrc) * kFinChunk + threadIdx.x;
        if (col < d.W) {
            const float* cp = ws + d.colpart + static_cast<int64_t>(b) * d.tr * d.W + col;
            double s = 0.0;
            for (int rt = 0; rt < d.tr; ++rt) s += static_cast<double>(ldf(cp + static_cast<int64_t>(rt) * d.W));
            float* dst = cs + static_cast<int64_t>(b) * d.W + col;
            const double mean = s / static_cast<double>(d.H);
            const double cnew = beta != 0.0 ? beta * static_cast<double>(ldf(dst)) + omb * mean : mean;
            stf(dst, static_cast<float>(cnew));
        }
    }
}

void launch_finalize(const Table& t, int64_t items, const FinArgs& a, hipStream_t s) {
    if (items > 0) hipLaunchKernelGGL(k_finalize, dim3(static_cast<uint32_t>(items)), dim3(kThreads), 0, s, t, a);
}

// ----------------------------------------------------------------------------- k_rms

__global__ __launch_bounds__(kThreads) void k_rms(Table t, int32_t need_x) {
    __shared__ float lds[2 * kWaves];
    const int64_t tile = blockIdx.x;
    const int k = tensor_of(t.tile_tensor, tile);
    const TDesc d = t.desc[k];
    if (!d.factored) return;  // flat tensors finished their sums in k_stats
    const int64_t lt = tile - d.tile0;
    const TileRC p = tile_rc(d, lt);
    const bool vec = d.vec, bf = d.gbf16;
    const float* ws = t.ws;
    const float sm = static_cast<float>(sqrt(row_mean(d, ws, p.b)));
    const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
    float cf[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e)
        cf[e] = e < p.valid ? rsqrtf(ldf(d.c + static_cast<int64_t>(p.b) * d.W + p.col + e)) : 0.0f;
    const float* rrow = d.r + static_cast<int64_t>(p.b) * d.H;
    float su[kVec], sx[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) { su[e] = 0.0f; sx[e] = 0.0f; }
    for (int i0 = 0; i0 < p.nrows; i0 += 8) {
        float g[8][kVec];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i0 + i < p.nrows)
                load_g8<true>(d.g, mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, bf, g[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i0 + i < p.nrows) {
                const float rf = rsqrtf(ldf(rrow + p.row0 + i0 + i)) * sm;
#pragma unroll
                for (int e = 0; e < kVec; ++e) {
                    const float u = (g[i][e] * cf[e]) * rf;
                    su[e] = fmaf(u, u, su[e]);
                }
            }
        }
        if (need_x) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                if (i0 + i < p.nrows) {
                    float x[kVec];
                    load_f8<true>(d.x + mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, x);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
                }
            }
        }
    }
    float tu = sum8(su), tx = sum8(sx);
    block_sum2(tu, tx, lds);
    if (threadIdx.x == 0) {
        float* tp = t.ws + d.tilepart + 2 * lt;
        stf(tp, tu);
        stf(tp + 1, tx);
    }
}

void launch_rms(const Table& t, int64_t tiles, int32_t need_x, hipStream_t s) {
    if (tiles > 0) hipLaunchKernelGGL(k_rms, dim3(static_cast<uint32_t>(tiles)), dim3(kThreads), 0, s, t, need_x);
}

// ----------------------------------------------------------------------------- k_scalars

// Sum over the tensor's tiles of tilepart[.][0] and [.][1], fp64, fixed order.
__device__ __forceinline__ void tile_sums(const TDesc& d, const float* __restrict__ ws, double& su,
                                          double& sx, double* lds) {
    double a = 0.0, b = 0.0;
    const float* tp = ws + d.tilepart;
    for (int j = threadIdx.x; j < d.ntiles; j += kThreads) {
        a += static_cast<double>(ldf(tp + 2 * j));
        b += static_cast<double>(ldf(tp + 2 * j + 1));
    }
    su = block_sum_d(a, lds);
    __syncthreads();
    sx = block_sum_d(b, lds + kWaves);
}

__global__ __launch_bounds__(kThreads) void k_scalars(Table t, ScalArgs a) {
    __shared__ double lds[2 * kWaves];
    const int k = blockIdx.x;
    const TDesc d = t.desc[k];
    if (d.numel == 0) return;
    float* ws = t.ws;
    float* scal = ws + d.scal;
    float* bs = ws + d.bscal;
    const int w = threadIdx.x >> 6;
    const double n = static_cast<double>(d.numel);

    if (a.mode == kScalCame2) {
        // Confidence statistic: per-matrix lr * sqrt(mean of its row statistic).
        if (!d.factored) return;
        for (int b = w; b < d.B; b += kWaves) {
            const double mr = row_mean(d, ws, b);
            if ((threadIdx.x & 63) == 0) stf(bs + d.B + b, static_cast<float>(a.lr * sqrt(mr)));
        }
        return;
    }

    double su, sx;
    tile_sums(d, ws, su, sx, lds);
    if (a.mode == kScalLamb) {
        // su: sum of x^2, sx: sum of d^2 (see the LAMB moment pass).
        const double xn = sqrt(su), dn = sqrt(sx);
        const double trust = (xn > 0.0 && dn > 0.0) ? xn / dn : 1.0;
        if (threadIdx.x == 0) {
            stf(bs + 0, static_cast<float>(a.lr * trust));
            stf(scal + kSlotRmsX, static_cast<float>(xn));
            stf(scal + kSlotNormD, static_cast<float>(dn));
        }
        return;
    }
    const double rms_u = sqrt(su / n);
    const double kappa = fmax(1.0, rms_u / a.clip);
    double alpha = 1.0;
    if (a.mode == kScalAdafactor) {
        const double rms_x = sqrt(sx / n);
        alpha = a.rho * (a.scale_parameter ? fmax(a.eps2, rms_x) : 1.0);
        if (threadIdx.x == 0) stf(scal + kSlotRmsX, static_cast<float>(rms_x));
    }
    const double coef = alpha / kappa;
    if (threadIdx.x == 0) {
        stf(scal + kSlotAlpha, static_cast<float>(alpha));
        stf(scal + kSlotCoef, static_cast<float>(coef));
        stf(scal + kSlotRmsU, static_cast<float>(rms_u));
        // Decoupled weight decay: Adafactor scales it by alpha, CAME by lr.
        stf(scal + kSlotDecay, static_cast<float>(a.mode == kScalAdafactor ? a.wd * alpha : a.wd * a.lr));
    }
    if (d.factored) {
        for (int b = w; b < d.B; b += kWaves) {
            const double mr = row_mean(d, ws, b);
            if ((threadIdx.x & 63) == 0) stf(bs + b, static_cast<float>(coef * sqrt(mr)));
        }
    } else if (threadIdx.x == 0) {
        stf(bs + 0, static_cast<float>(coef));
    }
}

void launch_scalars(const Table& t, int32_t n, const ScalArgs& a, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_scalars, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, a);
}

}  // namespace meo
