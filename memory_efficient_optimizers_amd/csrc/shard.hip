// Row-sharded steps: the partial sums one rank contributes, and the fold of their
// totals (summed over ranks by the caller) into the replicated column statistic.
//
// Each rank holds whole rows of a factored tensor, so the row-complete first pass
// runs unchanged on its rows: the row statistic R_i is final, and each strip leaves
// column sums of Q = G^2 + eps1 and S = G^2 / R_i and the sum of its new R_i. What
// the rank cannot finish is what needs every row: the column statistic C_j (mean of
// Q over all rows), mean(R), and through the identity
// sum_ij U_ij^2 = mean(R) * sum_j S_j / C_j the RMS of the update. Those are sums,
// so one all-reduce of the per-tensor records below finishes them on every rank.
#include "internal.h"

namespace meo {

// Items: a factored tensor's matrix b and 256-column chunk (b * chunks + chunk); a
// flat tensor, item 0. Writes the tensor's record (layout in meo.h). `carried`
// (Adafactor): the record's sum of X^2 is the shard's carried value (TDesc::xsq),
// which the previous step's apply pass formed from the rows it stored.
__global__ __launch_bounds__(kThreads) void k_shard_partials(Table t, float* partials, int32_t need_x,
                                                             int32_t carried) {
    __shared__ double lds[kWaves];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const float* ws = t.ws;
    float* out = partials + d.part;
    const int tid = threadIdx.x;
    if (d.mode == kFlat) {
        // Per-tile pairs of the first pass: (sum U^2, sum X^2) for Adafactor, (sum X^2,
        // sum d^2) for LAMB's moment pass.
        const float* tp = ws + d.tilepart;
        double s0 = 0.0, s1 = 0.0;
        for (int j = tid; j < d.tc; j += kThreads) {
            s0 += static_cast<double>(ldf(tp + 2 * j));
            s1 += static_cast<double>(ldf(tp + 2 * j + 1));
        }
        s0 = block_sum_d(s0, lds);
        __syncthreads();
        s1 = block_sum_d(s1, lds);
        if (carried && d.xsq) s1 = static_cast<double>(ldf(d.xsq));
        if (tid == 0) {
            stf(out, static_cast<float>(s0));
            stf(out + 1, static_cast<float>(s1));
        }
        return;
    }
    const int chunks = (d.W + kThreads - 1) / kThreads;
    const int b = it.y / chunks, ch = it.y - b * chunks;
    const int col = ch * kThreads + tid;
    const int64_t BW = static_cast<int64_t>(d.B) * d.W;
    if (col < d.W) {
        const float* cp = ws + d.colpart + static_cast<int64_t>(b) * d.strips * 2 * d.W + col;
        double q = 0.0, g = 0.0;
        for (int st = 0; st < d.strips; ++st) {
            q += static_cast<double>(ldf(cp + static_cast<int64_t>(st) * 2 * d.W));
            g += static_cast<double>(ldf(cp + static_cast<int64_t>(st) * 2 * d.W + d.W));
        }
        stf(out + static_cast<int64_t>(b) * d.W + col, static_cast<float>(q));
        stf(out + BW + static_cast<int64_t>(b) * d.W + col, static_cast<float>(g));
    }
    if (ch == 0) {  // block-uniform
        const float* tp = ws + d.tilepart + 2 * static_cast<int64_t>(b) * d.strips;
        double r = 0.0;
        for (int st = tid; st < d.strips; st += kThreads) r += static_cast<double>(ldf(tp + 2 * st));
        r = block_sum_d(r, lds);
        __syncthreads();
        if (tid == 0) stf(out + 2 * BW + b, static_cast<float>(r));
        if (b == 0) {
            double x = 0.0;
            if (need_x)  // the sum(X^2) chunks ran only then
                for (int j = tid; j < d.xchunks; j += kThreads) x += static_cast<double>(ldf(ws + d.xpart + j));
            x = block_sum_d(x, lds);
            if (carried && d.xsq) x = static_cast<double>(ldf(d.xsq));
            if (tid == 0) stf(out + 2 * BW + d.B, static_cast<float>(x));
        }
    }
}

void launch_shard_partials(const Table& t, int64_t n, float* partials, int32_t need_x, int32_t carried,
                           hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_shard_partials, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, partials,
                                  need_x, carried);
}

// Items: a factored tensor's matrix b and 256-column chunk. From the totals: C_j <-
// beta C_j + (1 - beta) (sum of Q_j over all rows) / H, and per 64-column chunk
// (one wave) the sum of S_j / C_j, written where the whole-tensor step's finalize
// pass leaves it (sumr[b][chunk]) for the scalar pass.
__global__ __launch_bounds__(kThreads) void k_shard_fold(Table t, const float* partials, double beta) {
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const int chunks = (d.W + kThreads - 1) / kThreads;
    const int b = it.y / chunks, ch = it.y - b * chunks;
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = ch * kThreads + threadIdx.x;
    const float* in = partials + d.part;
    const int64_t BW = static_cast<int64_t>(d.B) * d.W;
    double u = 0.0;
    if (col < d.W) {
        float* dst = d.c + static_cast<int64_t>(b) * d.W + col;
        const double mean = static_cast<double>(ldf(in + static_cast<int64_t>(b) * d.W + col)) /
                            static_cast<double>(d.total);
        const double cnew = beta != 0.0 ? beta * static_cast<double>(ldf(dst)) + (1.0 - beta) * mean : mean;
        const float c32 = static_cast<float>(cnew);
        stf(dst, c32);
        u = static_cast<double>(ldf(in + BW + static_cast<int64_t>(b) * d.W + col)) / static_cast<double>(c32);
    }
    u = wave_sum(u);
    const int cj = ch * kWaves + w;  // 64-column chunk of this wave
    if (lane == 0 && cj < d.ncc) stf(t.ws + d.sumr + static_cast<int64_t>(b) * d.ncc + cj, static_cast<float>(u));
}

void launch_shard_fold(const Table& t, int64_t n, const float* partials, double beta, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_shard_fold, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, partials,
                                  beta);
}

// CAME, after the moment pass on the shard's rows: items (tensor, matrix b and
// 256-column chunk). Column sums of E = (U - M)^2 + eps2 over the shard's row tiles,
// and (chunk 0) the sum of the new confidence row statistic, which the finalize
// pass left per 256-row chunk in sumr. Record: [B][W] sums of E, [B] sums of Rr.
__global__ __launch_bounds__(kThreads) void k_conf_partials(Table t, float* conf) {
    __shared__ double lds[kWaves];
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const float* ws = t.ws;
    float* out = conf + d.part2;
    const int chunks = (d.W + kThreads - 1) / kThreads;
    const int b = it.y / chunks, ch = it.y - b * chunks;
    const int col = ch * kThreads + threadIdx.x;
    if (col < d.W) {
        const float* cp = ws + d.colpart + static_cast<int64_t>(b) * d.tr * d.W + col;
        double e = 0.0;
        for (int rt = 0; rt < d.tr; ++rt) e += static_cast<double>(ldf(cp + static_cast<int64_t>(rt) * d.W));
        stf(out + static_cast<int64_t>(b) * d.W + col, static_cast<float>(e));
    }
    if (ch == 0) {  // block-uniform
        const float* sr = ws + d.sumr + static_cast<int64_t>(b) * d.nrc;
        double r = 0.0;
        for (int j = threadIdx.x; j < d.nrc; j += kThreads) r += static_cast<double>(ldf(sr + j));
        r = block_sum_d(r, lds);
        if (threadIdx.x == 0) stf(out + static_cast<int64_t>(d.B) * d.W + b, static_cast<float>(r));
    }
}

void launch_conf_partials(const Table& t, int64_t n, float* conf, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_conf_partials, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, conf);
}

// CAME, from the confidence totals: Rc_j <- beta3 Rc_j + (1 - beta3) (sum of E_j
// over all rows) / H.
__global__ __launch_bounds__(kThreads) void k_conf_fold(Table t, const float* conf, double beta) {
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const int chunks = (d.W + kThreads - 1) / kThreads;
    const int b = it.y / chunks, ch = it.y - b * chunks;
    const int col = ch * kThreads + threadIdx.x;
    if (col >= d.W) return;
    float* dst = d.rc + static_cast<int64_t>(b) * d.W + col;
    const double mean = static_cast<double>(ldf(conf + d.part2 + static_cast<int64_t>(b) * d.W + col)) /
                        static_cast<double>(d.total);
    const double cnew = beta != 0.0 ? beta * static_cast<double>(ldf(dst)) + (1.0 - beta) * mean : mean;
    stf(dst, static_cast<float>(cnew));
}

void launch_conf_fold(const Table& t, int64_t n, const float* conf, double beta, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_conf_fold, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, conf, beta);
}

__global__ __launch_bounds__(kThreads) void k_zero_records(const int2* items, float* partials) {
    const int2 r = items[blockIdx.x];
    for (int i = threadIdx.x; i < r.y; i += kThreads) stf(partials + r.x + i, 0.0f);
}

void launch_zero_records(const int2* items, int64_t n, float* partials, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_zero_records, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, items, partials);
}

}  // namespace meo
