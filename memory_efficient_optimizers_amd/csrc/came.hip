// CAME passes beyond the shared Adafactor-style statistics.
//
// The page (Colossal-AI distributed optimizers, "four optimizers" table and the
// DistributedCAME paragraph) describes CAME as Adafactor's factorisation plus a
// confidence matrix tracked with a third beta; the step order is that of the CAME
// paper it cites (arXiv:2307.02047):
//
//   k_came_mom    u = G / sqrt(V_hat) / kappa (rebuilt on the fly),
//                 M <- beta1 M + (1 - beta1) u, stored;
//                 factored: row and column sums of E = (u - M)^2 + eps2 per tile
//                 (the instability), folded into the confidence statistics by the
//                 shared finalize pass with beta3;
//                 1-D: the step is M itself, X <- X - lr wd X - lr M.
//   k_came_apply  factored: X <- X - lr wd X - M * rsqrt(S_ij) * lr with
//                 S_ij = Rs_i Cs_j / mean(Rs) rebuilt on the fly.
#include "internal.h"

namespace meo {

template <int ST>
__global__ __launch_bounds__(kThreads) void k_came_mom(Table t, CameArgs a) {
    __shared__ __align__(16) float lds[kWaves * kTileCols];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of an XCD-aligned list
    const TDesc d = t.desc[it.x];
    const int lt = it.y;
    float* ws = t.ws;
    const bool vec = d.vec, bf = d.gbf16, xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    const float b1 = a.beta1, omb1 = a.omb1;

    if (d.mode != kFlat) {
        const TileRC p = tile_rc(d, lt);
        const int lane = threadIdx.x & 63;
        const float coef = ldf(ws + d.bscal + p.b);
        const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
        float cf[kVec], cs[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            cf[e] = e < p.valid ? rsqrtf(ldf(d.c + static_cast<int64_t>(p.b) * d.W + p.col + e)) : 0.0f;
            cs[e] = 0.0f;
        }
        const float* rrow = d.r + static_cast<int64_t>(p.b) * d.H;
        float* rowpart = ws + d.rowpart + (static_cast<int64_t>(p.b) * d.tc + p.ct) * d.H;
        // 2 rows per batch with an 8-bit first moment (registers of its
        // re-quantization), 4 otherwise.
        constexpr int RB = (ST == kStoreF32I8 || ST == kStoreBf16I8) ? 2 : 4;
        for (int i0 = 0; i0 < p.nrows; i0 += RB) {
            float g[RB][kVec], m[RB][kVec];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i0 + i < p.nrows) {
                    const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                    load_v8(d.g, off, p.valid, vec, bf, g[i]);
                    load_m8(d, off, p.valid, vec, mb, mi, m[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i0 + i < p.nrows) {
                    const int row = p.row0 + i0 + i;
                    const int64_t off = mat + static_cast<int64_t>(row) * d.W + p.col;
                    const float rf = rsqrtf(ldf(rrow + row)) * coef;
                    float u[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        u[e] = (g[i][e] * cf[e]) * rf;
                        m[i][e] = fmaf(b1, m[i][e], omb1 * u[e]);
                    }
                    Q8 qm;
                    settle_m8(m[i], mb, mi, qm);  // the instability uses the stored moment
                    float rs = 0.0f;
#pragma unroll
                    for (int e = 0; e < kVec; ++e) {
                        const float du = u[e] - m[i][e];
                        const float q = e < p.valid ? fmaf(du, du, a.eps2) : 0.0f;
                        cs[e] += q;
                        rs += q;
                    }
                    store_m8(d, off, p.valid, vec, mb, mi, m[i], qm);
                    rs = wave_sum(rs);
                    if (lane == 0) stf(rowpart + row, rs);
                }
            }
        }
        write_colpart(d, ws, p, cs, lds);
    } else {
        const float coef = ldf(ws + d.bscal);
        const float decay = ldf(ws + d.scal + kSlotDecay);
        const float lr = a.lr;
        const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
        for (int it = 0; it < kFlatIters; ++it) {
            // Block-uniform exit (cross-lane work of an 8-bit first moment).
            if (base + static_cast<int64_t>(it) * kThreads * kVec >= d.numel) break;
            const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
            const int valid = clamp_valid(d.numel - i);
            float g[kVec], v[kVec], x[kVec], m[kVec];
            load_v8(d.g, i, valid, vec, bf, g);
            load_f8(d.v + i, valid, vec, v);
            load_v8(d.x, i, valid, vec, xb, x);
            load_m8(d, i, valid, vec, mb, mi, m);
#pragma unroll
            for (int e = 0; e < kVec; ++e) {
                const float u = e < valid ? (g[e] * rsqrtf(v[e])) * coef : 0.0f;
                m[e] = fmaf(b1, m[e], omb1 * u);
            }
            Q8 qm;
            settle_m8(m, mb, mi, qm);  // the step is the stored moment
#pragma unroll
            for (int e = 0; e < kVec; ++e) x[e] = fmaf(-decay, x[e], x[e]) - lr * m[e];
            store_m8(d, i, valid, vec, mb, mi, m, qm);
            store_v8(d.x, i, valid, vec, xb, x);
        }
    }
}

void launch_came_mom(const Table& t, int64_t n, const CameArgs& a, int storage, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (storage == kStoreF32) hipLaunchKernelGGL(k_came_mom<kStoreF32>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16) hipLaunchKernelGGL(k_came_mom<kStoreBf16>, grid, block, 0, s, t, a);
    else if (storage == kStoreF32I8) hipLaunchKernelGGL(k_came_mom<kStoreF32I8>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16I8) hipLaunchKernelGGL(k_came_mom<kStoreBf16I8>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_came_mom<kStoreMixed>, grid, block, 0, s, t, a);
}

template <int ST>
__global__ __launch_bounds__(kThreads) void k_came_apply(Table t) {
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of an XCD-aligned list
    const TDesc d = t.desc[it.x];
    if (d.mode == kFlat) return;  // 1-D tensors were finished by k_came_mom
    const int lt = it.y;
    const float* ws = t.ws;
    const bool vec = d.vec, xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    const TileRC p = tile_rc(d, lt);
    const float coef = ldf(ws + d.bscal + d.B + p.b);
    const float decay = ldf(ws + d.scal + kSlotDecay);
    const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
    float sc[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e)
        sc[e] = e < p.valid ? rsqrtf(ldf(d.rc + static_cast<int64_t>(p.b) * d.W + p.col + e)) : 0.0f;
    const float* rrow = d.rr + static_cast<int64_t>(p.b) * d.H;
    for (int i0 = 0; i0 < p.nrows; i0 += 4) {
        float x[4][kVec], m[4][kVec];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i0 + i < p.nrows) {
                const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                load_v8(d.x, off, p.valid, vec, xb, x[i]);
                load_m8(d, off, p.valid, vec, mb, mi, m[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (i0 + i < p.nrows) {
                const int row = p.row0 + i0 + i;
                const int64_t off = mat + static_cast<int64_t>(row) * d.W + p.col;
                const float sr = rsqrtf(ldf(rrow + row)) * coef;
#pragma unroll
                for (int e = 0; e < kVec; ++e) x[i][e] = fmaf(-decay, x[i][e], x[i][e]) - (m[i][e] * sc[e]) * sr;
                store_v8(d.x, off, p.valid, vec, xb, x[i]);
            }
        }
    }
}

void launch_came_apply(const Table& t, int64_t n, int storage, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (storage == kStoreF32) hipLaunchKernelGGL(k_came_apply<kStoreF32>, grid, block, 0, s, t);
    else if (storage == kStoreBf16) hipLaunchKernelGGL(k_came_apply<kStoreBf16>, grid, block, 0, s, t);
    else if (storage == kStoreF32I8) hipLaunchKernelGGL(k_came_apply<kStoreF32I8>, grid, block, 0, s, t);
    else if (storage == kStoreBf16I8) hipLaunchKernelGGL(k_came_apply<kStoreBf16I8>, grid, block, 0, s, t);
    else hipLaunchKernelGGL(k_came_apply<kStoreMixed>, grid, block, 0, s, t);
}

}  // namespace meo
