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
//                 S_ij = Rs_i Cs_j / mean(Rs) rebuilt on the fly; one item per
//                 kFlatTile elements in memory order (aligned rows) or per 64 x 512
//                 tile (other rows).
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

// Factored tensors with 16-byte aligned rows (W % 8 == 0): item lt covers elements
// [lt * kFlatTile, (lt + 1) * kFlatTile) of the tensor in memory order, and each
// lane's 8 elements (one row, since W % 8 == 0) find their row and column from their
// index. At every batch the block's four waves then load one contiguous 8 KB range
// per stream, where 64 x 512 tiles load 2 KB pieces of 16 rows; the pass runs about
// 5% faster so (Llama-7B list). The arithmetic is the tiled path's, term for term.
template <int ST, typename I>
__device__ __forceinline__ void came_apply_range(const TDesc& d, int lt, const float* ws, float decay) {
    const I W = static_cast<I>(d.W), H = static_cast<I>(d.H);
    const I numel = static_cast<I>(d.B) * H * W;
    const I base = static_cast<I>(lt) * kFlatTile;
    const bool xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    constexpr int RB = 4;  // groups of 8 per lane in flight
    for (int j0 = 0; j0 < kFlatIters; j0 += RB) {
        float x[RB][kVec], m[RB][kVec];
        I ix[RB];
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            ix[j] = base + (static_cast<I>(j0 + j) * kThreads + threadIdx.x) * kVec;
            if (ix[j] < numel) {
                load_v8(d.x, ix[j], kVec, true, xb, x[j]);
                load_m8(d, ix[j], kVec, true, mb, mi, m[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < RB; ++j) {
            if (ix[j] < numel) {
                const I rg = ix[j] / W;  // row over all B matrices
                const I col = ix[j] - rg * W;
                const I b = rg / H;
                const float sr = rsqrtf(ldf(d.rr + rg)) * ldf(ws + d.bscal + d.B + b);
                const float* rc = d.rc + b * W + col;
#pragma unroll
                for (int e = 0; e < kVec; ++e)
                    x[j][e] = fmaf(-decay, x[j][e], x[j][e]) - (m[j][e] * rsqrtf(ldf(rc + e))) * sr;
                store_v8(d.x, ix[j], kVec, true, xb, x[j]);
            }
        }
    }
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
    const float decay = ldf(ws + d.scal + kSlotDecay);
    if (vec) {
        // 32-bit index arithmetic while the tensor has fewer than 2^32 elements
        if (static_cast<int64_t>(d.B) * d.H * d.W < (int64_t{1} << 32))
            came_apply_range<ST, uint32_t>(d, lt, ws, decay);
        else
            came_apply_range<ST, uint64_t>(d, lt, ws, decay);
        return;
    }
    // Rows that are not 16-byte aligned: 64 x 512 tiles, element-wise accesses.
    const TileRC p = tile_rc(d, lt);
    const float coef = ldf(ws + d.bscal + d.B + p.b);
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
