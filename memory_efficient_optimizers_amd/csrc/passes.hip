// Passes shared by Adafactor and CAME (and the scalar pass shared with LAMB).
//
// The factored statistics follow the "four optimizers" table of the Colossal-AI
// distributed-optimizers page (second moment approximated by row * col) and its
// section "Step 3" (row statistic [H], column statistic [W], full statistic for
// 1-D tensors); RMS clipping and the step-size rules follow the note after its
// "Step 5". With Q = G^2 + eps1, R_i = mean_j Q_ij, C_j = mean_i Q_ij (EMA'd) and
// V_ij = R_i C_j / mean(R), the update U = G / sqrt(V) has
//     sum U^2 = mean(R) * sum_j S_j / C_j,   S_j = sum_i G_ij^2 / R_i,
// which is what lets a single read of G give both statistics and RMS(U) once a
// block holds whole rows.
//
//   k_rowstats0/1  row-complete tensors: one read of G per strip of full rows:
//                  new R_i (stored), per-strip column sums of Q and of G^2 / R_i
//                  and the strip's sum of R_i. Flat tensors (with class 0):
//                  V <- beta V + (1-beta) Q, sums of G^2 / V and X^2.
//   k_xnorm        row-complete tensors (Adafactor): sum(X^2) per chunk of X.
//   k_stats        tiled tensors: per-tile row sums and column sums of Q.
//   k_finalize     column (and, tiled, row) statistics from the partials in fp64,
//                  fixed order; row-complete: per-chunk sums of S_j / C_j;
//                  tiled: per-chunk sums of the new row statistic.
//   k_rms          tiled tensors only: second read of G (and X) for sum U^2, X^2.
//   k_scalars      one block per tensor: RMS(U), RMS(X), the clip divisor, alpha
//                  and the per-matrix coefficients of the apply passes.
#include "internal.h"

namespace meo {

// ----------------------------------------------------------------------------- flat first pass

// Block of NTHR threads over one flat tile of kFlatTile elements; `lds` holds
// 2 * NTHR / 64 floats.
template <int NTHR>
__device__ void stats_flat(const TDesc& d, int lt, float* __restrict__ ws, const StatsArgs& a, float* lds) {
    constexpr int ITERS = kFlatTile / (NTHR * kVec);
    const bool vec = d.vec, bf = d.gbf16;
    const float beta = a.beta, omb = a.omb;
    const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
    float su[kVec], sx[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) { su[e] = 0.0f; sx[e] = 0.0f; }
    for (int it = 0; it < ITERS; ++it) {
        const int64_t i = base + (static_cast<int64_t>(it) * NTHR + threadIdx.x) * kVec;
        const int valid = clamp_valid(d.numel - i);
        if (valid == 0) break;
        float g[kVec], v[kVec] = {};
        load_v8<true>(d.g, i, valid, vec, bf, g);
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
            load_v8<true>(d.x, i, valid, vec, d.xbf16, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
        }
    }
    float tu = sum8(su), tx = sum8(sx);
    block_sum2<NTHR / kLanes>(tu, tx, lds);
    if (threadIdx.x == 0) {
        float* tp = ws + d.tilepart + 2 * static_cast<int64_t>(lt);
        stf(tp, tu);
        stf(tp + 1, tx);
    }
}

// ----------------------------------------------------------------------------- sum of X^2 chunks

// Sum of X^2 over chunk `c` (kFlatTile elements) of a row-complete tensor's
// parameter. These blocks run as a grid of their own: with few registers, 8 waves
// per SIMD keep the loads in flight. Interleaved with the strips in one grid they
// ran at the strips' 3 waves per SIMD, and the two streams together took 1.2 ms
// longer than apart on the 7B list.
template <int NTHR>
__device__ void xnorm_chunk(const TDesc& d, int c, float* __restrict__ ws, const StatsArgs& a, float* bsum) {
    if (!a.need_x) return;  // the step does not use RMS(X)
    constexpr int NW = NTHR / kLanes;
    constexpr int ITERS = kFlatTile / (NTHR * kVec);
    const int64_t base = static_cast<int64_t>(c) * kFlatTile;
    float sx[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) sx[e] = 0.0f;
    if (d.xbf16 && base + kFlatTile <= d.numel) {
        // A whole bf16 chunk: half the bytes of fp32 per element, so all of the
        // thread's 16-byte loads are issued before the first is used.
        const uint16_t* xp = static_cast<const uint16_t*>(d.x) + base + threadIdx.x * kVec;
        u32x4 raw[ITERS];
#pragma unroll
        for (int it = 0; it < ITERS; ++it) raw[it] = ld_u4<true>(xp + static_cast<int64_t>(it) * NTHR * kVec);
#pragma unroll
        for (int it = 0; it < ITERS; ++it) {
            float x[kVec];
            bf16x8(raw[it], x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
        }
    } else {
#pragma unroll 8
        for (int it = 0; it < ITERS; ++it) {
            const int64_t i = base + (static_cast<int64_t>(it) * NTHR + threadIdx.x) * kVec;
            const int valid = clamp_valid(d.numel - i);
            if (valid == 0) break;
            float x[kVec];
            load_v8<true>(d.x, i, valid, true, d.xbf16, x);
#pragma unroll
            for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
        }
    }
    float tx = sum8(sx), unused = 0.0f;
    block_sum2<NW>(tx, unused, bsum);
    if (threadIdx.x == 0) stf(ws + d.xpart + c, tx);
}

// ----------------------------------------------------------------------------- row-complete first pass

// Raw gradient of one batch of rows: per 8-column group one u32x4 (bf16) or two
// (fp32, reinterpreted).
template <int RB, int KMAX, bool BF16>
struct GBatch {
    u32x4 v[RB][KMAX][BF16 ? 1 : 2];
};

template <int NTHR, int RB, int KMAX, bool BF16>
__device__ __forceinline__ void load_batch(GBatch<RB, KMAX, BF16>& gb, const void* g, int64_t mat, int r0,
                                           int nr, int W, int ngroups) {
#pragma unroll
    for (int r = 0; r < RB; ++r)
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            const int grp = threadIdx.x + k * NTHR;
            if (r < nr && grp < ngroups) {
                const int64_t off = mat + static_cast<int64_t>(r0 + r) * W + grp * kVec;
                if (BF16) {
                    gb.v[r][k][0] = ld_u4<true>(static_cast<const uint16_t*>(g) + off);
                } else {
                    gb.v[r][k][0] = ld_u4<true>(static_cast<const float*>(g) + off);
                    gb.v[r][k][BF16 ? 0 : 1] = ld_u4<true>(static_cast<const float*>(g) + off + 4);
                }
            }
        }
}

template <int RB, int KMAX, bool BF16>
__device__ __forceinline__ void unpack(const GBatch<RB, KMAX, BF16>& gb, int r, int k, float* g) {
    if (BF16) {
        bf16x8(gb.v[r][k][0], g);
    } else {
        const u32x4 a = gb.v[r][k][0], b = gb.v[r][k][BF16 ? 0 : 1];
        g[0] = __uint_as_float(a.x); g[1] = __uint_as_float(a.y); g[2] = __uint_as_float(a.z); g[3] = __uint_as_float(a.w);
        g[4] = __uint_as_float(b.x); g[5] = __uint_as_float(b.y); g[6] = __uint_as_float(b.z); g[7] = __uint_as_float(b.w);
    }
}

// State of one strip while its batches go by.
struct StripCtx {
    int64_t mat;
    int row_begin, row_end, W, ngroups;
    float* rstat;
    float rsum;  // thread r < RB: sum of the new R over the rows it stored
};

// One batch of RB rows held in `cur`: row sums (lane partials, wave tree, waves in
// order through LDS slot `par`), the next batch's loads into `nxt`, one barrier,
// then every thread finishes the batch's row statistics from LDS and accumulates
// the column sums of Q and of G^2 / R_i.
template <int NTHR, int KMAX, int RB, bool BF16>
__device__ __forceinline__ void strip_batch(const TDesc& d, const StatsArgs& a, StripCtx& c, int r0, int par,
                                            const GBatch<RB, KMAX, BF16>& cur, GBatch<RB, KMAX, BF16>& nxt,
                                            float (&cs)[KMAX][kVec], float (&ss)[KMAX][kVec], float* red,
                                            const float* rold) {
    constexpr int NW = NTHR / kLanes;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int nr = min(RB, c.row_end - r0);
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        float acc[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) acc[e] = 0.0f;
#pragma unroll
        for (int k = 0; k < KMAX; ++k) {
            if (r < nr && tid + k * NTHR < c.ngroups) {
                float g[kVec];
                unpack<RB, KMAX, BF16>(cur, r, k, g);
#pragma unroll
                for (int e = 0; e < kVec; ++e) acc[e] += fmaf(g[e], g[e], a.eps1);
            }
        }
        const float rs = wave_sum(sum8(acc));
        if (lane == 0) red[(par * NW + w) * RB + r] = rs;
    }
    const int rn = r0 + RB;
    if (rn < c.row_end) load_batch<NTHR, RB, KMAX, BF16>(nxt, d.g, c.mat, rn, min(RB, c.row_end - rn), c.W, c.ngroups);
    __syncthreads();
    float ri[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        ri[r] = 0.0f;
        if (r < nr) {
            float tot = red[(par * NW) * RB + r];
#pragma unroll
            for (int i = 1; i < NW; ++i) tot += red[(par * NW + i) * RB + r];
            const double mean = static_cast<double>(tot) / static_cast<double>(c.W);
            const double rnew = a.beta != 0.0f
                                    ? a.dbeta * static_cast<double>(rold[r0 - c.row_begin + r]) + a.domb * mean
                                    : mean;
            const float r32 = static_cast<float>(rnew);
            ri[r] = 1.0f / r32;
            if (tid == r) {
                stf(c.rstat + r0 + r, r32);
                c.rsum += r32;
            }
        }
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
        if (r < nr) {
#pragma unroll
            for (int k = 0; k < KMAX; ++k) {
                if (tid + k * NTHR < c.ngroups) {
                    float g[kVec];
                    unpack<RB, KMAX, BF16>(cur, r, k, g);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        cs[k][e] += fmaf(g[e], g[e], a.eps1);
                        ss[k][e] = fmaf(g[e] * g[e], ri[r], ss[k][e]);
                    }
                }
            }
        }
    }
}

// One strip of up to d.srows full rows of matrix b (the sum of X^2 is taken by
// k_xnorm). Thread t owns the 8-column groups t,
// t + NTHR, ..., t + (KMAX-1) NTHR; rows go in batches of RB, two register buffers
// alternating so that a batch's loads are in flight during the previous one's
// reduction. `red` holds 2 * NW * RB floats, `rold` kStripRowsMax.
template <int NTHR, int KMAX, int RB, bool BF16>
__device__ void rowstats_strip(const TDesc& d, int lt, float* __restrict__ ws, const StatsArgs& a, float* red,
                               float* rold, float* bsum) {
    constexpr int NW = NTHR / kLanes;
    const int tid = threadIdx.x;
    const int b = lt / d.strips;
    const int st = lt - b * d.strips;
    StripCtx c;
    c.row_begin = st * d.srows;
    c.row_end = min(c.row_begin + d.srows, d.H);
    c.W = d.W;
    c.ngroups = d.W / kVec;
    c.mat = static_cast<int64_t>(b) * d.H * d.W;
    c.rstat = d.r + static_cast<int64_t>(b) * d.H;
    c.rsum = 0.0f;
    if (a.beta != 0.0f && tid < c.row_end - c.row_begin) rold[tid] = ldf(c.rstat + c.row_begin + tid);

    float cs[KMAX][kVec], ss[KMAX][kVec];
#pragma unroll
    for (int k = 0; k < KMAX; ++k)
#pragma unroll
        for (int e = 0; e < kVec; ++e) { cs[k][e] = 0.0f; ss[k][e] = 0.0f; }

    GBatch<RB, KMAX, BF16> b0, b1;
    load_batch<NTHR, RB, KMAX, BF16>(b0, d.g, c.mat, c.row_begin, min(RB, c.row_end - c.row_begin), c.W, c.ngroups);
    for (int r0 = c.row_begin; r0 < c.row_end; r0 += 2 * RB) {
        strip_batch<NTHR, KMAX, RB, BF16>(d, a, c, r0, 0, b0, b1, cs, ss, red, rold);
        if (r0 + RB < c.row_end) strip_batch<NTHR, KMAX, RB, BF16>(d, a, c, r0 + RB, 1, b1, b0, cs, ss, red, rold);
    }
    // Per-strip column partials: colpart[b][st][0][:] = sum Q, [1][:] = sum G^2 / R.
    float* cp = ws + d.colpart + (static_cast<int64_t>(b) * d.strips + st) * 2 * c.W;
#pragma unroll
    for (int k = 0; k < KMAX; ++k) {
        const int grp = tid + k * NTHR;
        if (grp < c.ngroups) {
            store_f8(cp + grp * kVec, kVec, true, cs[k]);
            store_f8(cp + c.W + grp * kVec, kVec, true, ss[k]);
        }
    }
    float tr_ = c.rsum, unused = 0.0f;
    block_sum2<NW>(tr_, unused, bsum);
    if (tid == 0) stf(ws + d.tilepart + 2 * static_cast<int64_t>(lt), tr_);
}

// Rows per batch of the two classes (bf16 gradients; fp32 ones take half as many,
// so that both keep the same number of gradient registers).
constexpr int kRb0 = 4, kRb1 = 2;

__global__ __launch_bounds__(256) void k_rowstats0(Table t, StatsArgs a) {
    __shared__ float red[2 * kWaves * kRb0], rold[kStripRowsMax], bsum[2 * kWaves];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    if (d.mode == kFlat) stats_flat<256>(d, it.y, t.ws, a, bsum);
    else if (d.gbf16) rowstats_strip<256, 2, kRb0, true>(d, it.y, t.ws, a, red, rold, bsum);
    else rowstats_strip<256, 2, kRb0 / 2, false>(d, it.y, t.ws, a, red, rold, bsum);
}

__global__ __launch_bounds__(512) void k_rowstats1(Table t, StatsArgs a) {
    __shared__ float red[2 * 8 * kRb1], rold[kStripRowsMax], bsum[2 * 8];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    if (d.gbf16) rowstats_strip<512, 3, kRb1, true>(d, it.y, t.ws, a, red, rold, bsum);
    else rowstats_strip<512, 3, kRb1 / 2, false>(d, it.y, t.ws, a, red, rold, bsum);
}

__global__ __launch_bounds__(256) void k_xnorm(Table t, StatsArgs a) {
    __shared__ float bsum[2 * kWaves];
    const int2 it = t.items[blockIdx.x];
    xnorm_chunk<256>(t.desc[it.x], it.y, t.ws, a, bsum);
}

void launch_xnorm(const Table& t, int64_t n, const StatsArgs& a, hipStream_t s) {
    if (n <= 0) return;
    hipLaunchKernelGGL(k_xnorm, dim3(static_cast<uint32_t>(n)), dim3(256), 0, s, t, a);
}

void launch_rowstats(int cls, const Table& t, int64_t n, const StatsArgs& a, hipStream_t s) {
    if (n <= 0) return;
    if (cls == 0) hipLaunchKernelGGL(k_rowstats0, dim3(static_cast<uint32_t>(n)), dim3(256), 0, s, t, a);
    else hipLaunchKernelGGL(k_rowstats1, dim3(static_cast<uint32_t>(n)), dim3(512), 0, s, t, a);
}

// ----------------------------------------------------------------------------- tiled first pass

__global__ __launch_bounds__(kThreads) void k_stats(Table t, StatsArgs a) {
    __shared__ __align__(16) float lds[kWaves * kTileCols];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    float* ws = t.ws;
    const TileRC p = tile_rc(d, it.y);
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
                load_v8<true>(d.g, mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, bf, g[i]);
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

void launch_stats(const Table& t, int64_t n, const StatsArgs& a, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_stats, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, a);
}

// ----------------------------------------------------------------------------- k_finalize

// Items per matrix b: row-complete (first statistic): ncc column chunks; tiled (or
// `tiled_all`): nrc row chunks (kFinChunk rows) then ncc column chunks
// (kFinCols columns). A column chunk is one column per lane, the strips (or row
// tiles) split across the 4 waves, combined in wave order.
__global__ __launch_bounds__(kThreads) void k_finalize(Table t, FinArgs a) {
    __shared__ double part[kWaves][kLanes][2];
    __shared__ double lds[kWaves];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    float* ws = t.ws;
    float* rs = a.which ? d.rr : d.r;
    float* cs = a.which ? d.rc : d.c;
    const double beta = a.beta, omb = 1.0 - a.beta;
    const bool rc = d.mode == kRowComplete && !a.tiled_all;
    const int per = rc ? d.ncc : d.nrc + d.ncc;
    const int b = it.y / per;
    const int j = it.y - b * per;
    if (!rc && j < d.nrc) {
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
        return;
    }
    const int cj = rc ? j : j - d.nrc;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = cj * kFinCols + lane;
    double sq = 0.0, sg = 0.0;
    if (col < d.W) {
        if (rc) {
            const float* cp = ws + d.colpart + static_cast<int64_t>(b) * d.strips * 2 * d.W + col;
#pragma unroll 4
            for (int st = w; st < d.strips; st += kWaves) {
                sq += static_cast<double>(ldf(cp + static_cast<int64_t>(st) * 2 * d.W));
                sg += static_cast<double>(ldf(cp + static_cast<int64_t>(st) * 2 * d.W + d.W));
            }
        } else {
            const float* cp = ws + d.colpart + static_cast<int64_t>(b) * d.tr * d.W + col;
#pragma unroll 4
            for (int rt = w; rt < d.tr; rt += kWaves) sq += static_cast<double>(ldf(cp + static_cast<int64_t>(rt) * d.W));
        }
    }
    part[w][lane][0] = sq;
    part[w][lane][1] = sg;
    __syncthreads();
    if (w != 0) return;
    double u = 0.0;
    if (col < d.W) {
        sq = (part[0][lane][0] + part[1][lane][0]) + (part[2][lane][0] + part[3][lane][0]);
        sg = (part[0][lane][1] + part[1][lane][1]) + (part[2][lane][1] + part[3][lane][1]);
        float* dst = cs + static_cast<int64_t>(b) * d.W + col;
        const double mean = sq / static_cast<double>(d.H);
        const double cnew = beta != 0.0 ? beta * static_cast<double>(ldf(dst)) + omb * mean : mean;
        const float c32 = static_cast<float>(cnew);
        stf(dst, c32);
        u = sg / static_cast<double>(c32);
    }
    if (rc) {
        u = wave_sum(u);
        if (lane == 0) stf(ws + d.sumr + static_cast<int64_t>(b) * d.ncc + cj, static_cast<float>(u));
    }
}

void launch_finalize(const Table& t, int64_t n, const FinArgs& a, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_finalize, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, a);
}

// ----------------------------------------------------------------------------- k_rms (tiled)

__global__ __launch_bounds__(kThreads) void k_rms(Table t, int32_t need_x) {
    __shared__ float lds[2 * kWaves];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const TileRC p = tile_rc(d, it.y);
    const bool vec = d.vec, bf = d.gbf16;
    const float* ws = t.ws;
    const float sm = static_cast<float>(sqrt(row_mean_tiled(d, ws, p.b)));
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
                load_v8<true>(d.g, mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, bf, g[i]);
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
                    load_v8<true>(d.x, mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col, p.valid, vec, d.xbf16, x);
#pragma unroll
                    for (int e = 0; e < kVec; ++e) sx[e] = fmaf(x[e], x[e], sx[e]);
                }
            }
        }
    }
    float tu = sum8(su), tx = sum8(sx);
    block_sum2<kWaves>(tu, tx, lds);
    if (threadIdx.x == 0) {
        float* tp = t.ws + d.tilepart + 2 * static_cast<int64_t>(it.y);
        stf(tp, tu);
        stf(tp + 1, tx);
    }
}

void launch_rms(const Table& t, int64_t n, int32_t need_x, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_rms, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, need_x);
}

// ----------------------------------------------------------------------------- k_scalars

// Sum over `count` tile partials (stride 2, component `comp`), fp64, fixed order;
// every thread gets the result. `lds` holds kWaves doubles.
__device__ __forceinline__ double tile_sum(const float* __restrict__ tp, int count, int comp, double* lds) {
    double a = 0.0;
    for (int j = threadIdx.x; j < count; j += kThreads) a += static_cast<double>(ldf(tp + 2 * j + comp));
    const double r = block_sum_d(a, lds);
    __syncthreads();
    return r;
}

__global__ __launch_bounds__(kThreads) void k_scalars(const TDesc* __restrict__ desc, float* ws, ScalArgs a) {
    __shared__ double lds[kWaves];
    __shared__ double wsum[kWaves];
    const int k = blockIdx.x;
    const TDesc d = desc[k];
    float* scal = ws + d.scal;
    float* bs = ws + d.bscal;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const double n = static_cast<double>(d.numel);
    const float* tp = ws + d.tilepart;

    if (a.mode == kScalCame2) {
        // Confidence statistic (tiled layout for every factored tensor): per-matrix
        // lr * sqrt(mean of its row statistic); in a row-sharded step the mean comes
        // from the reduced confidence record (a.partials). The decay is written again
        // so that the apply pass needs nothing from an earlier call.
        if (d.mode == kFlat) return;
        if (threadIdx.x == 0) stf(scal + kSlotDecay, static_cast<float>(a.wd * a.lr));
        const float* P2 = a.partials ? a.partials + d.part2 : nullptr;
        for (int b = w; b < d.B; b += kWaves) {
            const double mr = P2 ? static_cast<double>(ldf(P2 + static_cast<int64_t>(d.B) * d.W + b)) /
                                       static_cast<double>(d.total)
                                 : row_mean_tiled(d, ws, b);
            if (lane == 0) stf(bs + d.B + b, static_cast<float>(a.lr * sqrt(mr)));
        }
        return;
    }
    // Row-sharded steps: the tensor's record of all-reduced partial sums.
    const float* P = a.partials ? a.partials + d.part : nullptr;
    if (a.mode == kScalLamb) {
        // components: sum of x^2, sum of d^2 (see the LAMB moment pass).
        const double xn = sqrt(P ? static_cast<double>(ldf(P)) : tile_sum(tp, d.tc, 0, lds));
        const double dn = sqrt(P ? static_cast<double>(ldf(P + 1)) : tile_sum(tp, d.tc, 1, lds));
        const double trust = (xn > 0.0 && dn > 0.0) ? xn / dn : 1.0;
        if (threadIdx.x == 0) {
            stf(bs, static_cast<float>(a.lr * trust));
            stf(scal + kSlotRmsX, static_cast<float>(xn));
            stf(scal + kSlotNormD, static_cast<float>(dn));
            stf(scal + kSlotTrust, static_cast<float>(trust));
        }
        return;
    }

    double su, sx;
    double numel = n;
    const int64_t BW = static_cast<int64_t>(d.B) * d.W;
    // mean of the new row statistic of matrix b
    auto row_mean = [&](int b) -> double {
        if (P) return static_cast<double>(ldf(P + 2 * BW + b)) / static_cast<double>(d.total);
        return d.mode == kRowComplete ? row_mean_rc(d, ws, b) : row_mean_tiled(d, ws, b);
    };
    if (P && d.mode == kFlat) {
        su = static_cast<double>(ldf(P));
        sx = static_cast<double>(ldf(P + 1));
        numel = static_cast<double>(d.total);
    } else if (d.mode == kRowComplete) {
        // sum U^2 = sum_b mean(R_b) * sum_j S_j / C_j (finalize chunk sums).
        double part = 0.0;
        for (int b = w; b < d.B; b += kWaves) {
            const double mr = row_mean(b);
            double u = 0.0;
            const float* sr = ws + d.sumr + static_cast<int64_t>(b) * d.ncc;
            for (int j = lane; j < d.ncc; j += kLanes) u += static_cast<double>(ldf(sr + j));
            part += mr * wave_sum(u);
        }
        if (lane == 0) wsum[w] = part;
        __syncthreads();
        su = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
        sx = 0.0;
        if (P) {
            sx = static_cast<double>(ldf(P + 2 * BW + d.B));
            numel = static_cast<double>(d.B) * static_cast<double>(d.total) * static_cast<double>(d.W);
        } else if (a.mode == kScalAdafactor && a.scale_parameter && !a.carried_x) {  // the chunks ran only then
            double a_ = 0.0;
            for (int j = threadIdx.x; j < d.xchunks; j += kThreads) a_ += static_cast<double>(ldf(ws + d.xpart + j));
            sx = block_sum_d(a_, lds);
            __syncthreads();
        }
    } else {
        const int tiles = d.mode == kFlat ? d.tc : d.B * d.tr * d.tc;
        su = tile_sum(tp, tiles, 0, lds);
        sx = tile_sum(tp, tiles, 1, lds);
    }
    // The carried sum of X^2: the previous step's apply pass summed the squares of
    // the parameter it stored, which is this step's pre-update parameter.
    if (a.carried_x && a.mode == kScalAdafactor && d.xsq) sx = static_cast<double>(ldf(d.xsq));
    const double rms_u = sqrt(su / numel);
    const double kappa = fmax(1.0, rms_u / a.clip);
    double alpha = 1.0;
    if (a.mode == kScalAdafactor) {
        const double rms_x = sqrt(sx / numel);
        alpha = a.rho * (a.scale_parameter ? fmax(a.eps2, rms_x) : 1.0);
        if (threadIdx.x == 0) stf(scal + kSlotRmsX, static_cast<float>(rms_x));
    }
    const double coef = alpha / kappa;
    if (threadIdx.x == 0) {
        stf(scal + kSlotAlpha, static_cast<float>(alpha));
        stf(scal + kSlotCoef, static_cast<float>(coef));
        stf(scal + kSlotRmsU, static_cast<float>(rms_u));
        stf(scal + kSlotKappa, static_cast<float>(kappa));
        // Decoupled weight decay: Adafactor scales it by alpha, CAME by lr.
        stf(scal + kSlotDecay, static_cast<float>(a.mode == kScalAdafactor ? a.wd * alpha : a.wd * a.lr));
    }
    if (d.mode == kFlat) {
        if (threadIdx.x == 0) stf(bs, static_cast<float>(coef));
        return;
    }
    for (int b = w; b < d.B; b += kWaves) {
        const double mr = row_mean(b);
        if (lane == 0) stf(bs + b, static_cast<float>(coef * sqrt(mr)));
    }
}

void launch_scalars(const TDesc* desc, float* ws, int32_t n, const ScalArgs& a, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_scalars, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, desc, ws, a);
}

// ----------------------------------------------------------------------------- carried sum(X^2)

// One block per tensor: the apply pass's per-tile sums of the updated X^2, in
// fp64 and a fixed order, into the tensor's carried value.
__global__ __launch_bounds__(kThreads) void k_sumsq_fold(const TDesc* __restrict__ desc, const float* ws) {
    __shared__ double lds[kWaves];
    const TDesc d = desc[blockIdx.x];
    if (!d.xsq) return;  // the whole block
    const int64_t tiles = d.mode == kFlat ? static_cast<int64_t>(d.tc)
                                          : static_cast<int64_t>(d.B) * d.tr * d.tc;
    double a = 0.0;
    for (int64_t j = threadIdx.x; j < tiles; j += kThreads) a += static_cast<double>(ldf(ws + d.apart + j));
    const double sum = block_sum_d(a, lds);
    if (threadIdx.x == 0) stf(d.xsq, static_cast<float>(sum));
}

void launch_sumsq_fold(const TDesc* desc, const float* ws, int32_t n, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_sumsq_fold, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, desc, ws);
}

}  // namespace meo
