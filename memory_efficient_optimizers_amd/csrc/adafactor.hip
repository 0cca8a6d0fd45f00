// Adafactor apply pass: the last streaming pass of the step.
//
// Per element: u = G * rsqrt(C_j) * rsqrt(R_i) * coef_b, where coef_b =
// sqrt(mean R of matrix b) * alpha / kappa (1-D tensors: u = G * rsqrt(V) * coef),
// i.e. the clipped, learning-rate-scaled update of the note after "Step 5" of the
// Colossal-AI distributed-optimizers page. With beta1 (page "Step 3": beta1 set ->
// exp_avg kept) M <- beta1 M + (1 - beta1) u and the step is M; otherwise the step
// is u. The parameter takes decoupled weight decay on its pre-update value:
// X <- X - (weight_decay * alpha) X - step.
#include "internal.h"

namespace meo {

__global__ __launch_bounds__(kThreads) void k_af_apply(Table t, AfApplyArgs a) {
    const int2 it = t.items[blockIdx.x];
    const TDesc d = t.desc[it.x];
    const int lt = it.y;
    const float* ws = t.ws;
    const float decay = ldf(ws + d.scal + kSlotDecay);
    const bool vec = d.vec, bf = d.gbf16, mom = a.has_beta1;
    const float b1 = a.beta1, omb1 = a.omb1;

    if (d.mode != kFlat) {
        const TileRC p = tile_rc(d, lt);
        const float coef = ldf(ws + d.bscal + p.b);
        const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
        float cf[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            cf[e] = e < p.valid ? rsqrtf(ldf(d.c + static_cast<int64_t>(p.b) * d.W + p.col + e)) : 0.0f;
        const float* rrow = d.r + static_cast<int64_t>(p.b) * d.H;
        for (int i0 = 0; i0 < p.nrows; i0 += 4) {
            float g[4][kVec], x[4][kVec], m[4][kVec];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i0 + i < p.nrows) {
                    const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                    load_g8(d.g, off, p.valid, vec, bf, g[i]);
                    load_f8(d.x + off, p.valid, vec, x[i]);
                    if (mom) load_f8(d.m + off, p.valid, vec, m[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i0 + i < p.nrows) {
                    const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                    const float rf = rsqrtf(ldf(rrow + p.row0 + i0 + i)) * coef;
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        const float u = (g[i][e] * cf[e]) * rf;
                        float step = u;
                        if (mom) {
                            m[i][e] = fmaf(b1, m[i][e], omb1 * u);
                            step = m[i][e];
                        }
                        x[i][e] = fmaf(-decay, x[i][e], x[i][e]) - step;
                    }
                    if (mom) store_f8(d.m + off, p.valid, vec, m[i]);
                    store_f8(d.x + off, p.valid, vec, x[i]);
                }
            }
        }
    } else {
        const float coef = ldf(ws + d.bscal);
        const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
        for (int it = 0; it < kFlatIters; ++it) {
            const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
            const int valid = clamp_valid(d.numel - i);
            if (valid == 0) break;
            float g[kVec], v[kVec], x[kVec], m[kVec] = {};
            load_g8(d.g, i, valid, vec, bf, g);
            load_f8(d.v + i, valid, vec, v);
            load_f8(d.x + i, valid, vec, x);
            if (mom) load_f8(d.m + i, valid, vec, m);
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const float u = e < valid ? (g[e] * rsqrtf(v[e])) * coef : 0.0f;
                float step = u;
                if (mom) {
                    m[e] = fmaf(b1, m[e], omb1 * u);
                    step = m[e];
                }
                x[e] = fmaf(-decay, x[e], x[e]) - step;
            }
            if (mom) store_f8(d.m + i, valid, vec, m);
            store_f8(d.x + i, valid, vec, x);
        }
    }
}

void launch_af_apply(const Table& t, int64_t n, const AfApplyArgs& a, hipStream_t s) {
    if (n > 0) hipLaunchKernelGGL(k_af_apply, dim3(static_cast<uint32_t>(n)), dim3(kThreads), 0, s, t, a);
}

}  // namespace meo
