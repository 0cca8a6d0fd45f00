// LAMB passes. The page (Colossal-AI distributed optimizers, "four optimizers"
// table and the DistributedLAMB paragraph) describes a layer-wise update scaled
// by a trust ratio of parameter and update norms; the per-tensor step is that of
// the LAMB paper it cites (arXiv:1904.00962):
//
//   k_lamb_moments  M <- b1 M + (1-b1) G, V <- b2 V + (1-b2) G^2 (stored);
//                   d = (M / bc1) / (sqrt(V / bc2) + eps) + wd X; per-tile sums of
//                   X^2 and d^2.
//   (k_scalars)     ratio = ||X|| / ||d|| (1 if either is 0), coef = lr * ratio.
//   k_lamb_apply    d recomputed from the stored M, V and X; X <- X - coef d.
//
// Every tensor is one flat layer, whatever its number of dims.
#include "internal.h"

namespace meo {

__device__ __forceinline__ float lamb_dir(float m, float v, float x, const LambArgs& a) {
    return (m * a.inv_bc1) / (sqrtf(v * a.inv_bc2) + a.eps) + a.wd * x;
}

template <int ST>
__global__ __launch_bounds__(kThreads) void k_lamb_moments(Table t, LambArgs a) {
    __shared__ float lds[2 * kWaves];
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of an XCD-aligned list
    const TDesc d = t.desc[it.x];
    const int lt = it.y;
    const bool vec = d.vec, bf = d.gbf16, xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
    float sx[kVec], sd[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) { sx[e] = 0.0f; sd[e] = 0.0f; }
    for (int it = 0; it < kFlatIters; ++it) {
        // Block-uniform exit (cross-lane work of an 8-bit first moment).
        if (base + static_cast<int64_t>(it) * kThreads * kVec >= d.numel) break;
        const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
        const int valid = clamp_valid(d.numel - i);
        float g[kVec], x[kVec], m[kVec], v[kVec];
        load_v8(d.g, i, valid, vec, bf, g);
        load_v8(d.x, i, valid, vec, xb, x);
        load_m8(d, i, valid, vec, mb, mi, m);
        load_f8(d.v + i, valid, vec, v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            m[e] = fmaf(a.beta1, m[e], a.omb1 * g[e]);
            v[e] = fmaf(a.beta2, v[e], a.omb2 * (g[e] * g[e]));
        }
        Q8 qm;
        settle_m8(m, mb, mi, qm);  // the direction uses the stored moment
#pragma unroll
        for (int e = 0; e < kVec; ++e) {
            const float dd = e < valid ? lamb_dir(m[e], v[e], x[e], a) : 0.0f;
            sx[e] = fmaf(x[e], x[e], sx[e]);
            sd[e] = fmaf(dd, dd, sd[e]);
        }
        store_m8(d, i, valid, vec, mb, mi, m, qm);
        store_f8(d.v + i, valid, vec, v);
    }
    float tx = sum8(sx), td = sum8(sd);
    block_sum2(tx, td, lds);
    if (threadIdx.x == 0) {
        float* tp = t.ws + d.tilepart + 2 * static_cast<int64_t>(lt);
        stf(tp, tx);
        stf(tp + 1, td);
    }
}

void launch_lamb_moments(const Table& t, int64_t n, const LambArgs& a, int storage, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (storage == kStoreF32) hipLaunchKernelGGL(k_lamb_moments<kStoreF32>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16) hipLaunchKernelGGL(k_lamb_moments<kStoreBf16>, grid, block, 0, s, t, a);
    else if (storage == kStoreF32I8) hipLaunchKernelGGL(k_lamb_moments<kStoreF32I8>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16I8) hipLaunchKernelGGL(k_lamb_moments<kStoreBf16I8>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_lamb_moments<kStoreMixed>, grid, block, 0, s, t, a);
}

template <int ST>
__global__ __launch_bounds__(kThreads) void k_lamb_apply(Table t, LambArgs a) {
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of an XCD-aligned list
    const TDesc d = t.desc[it.x];
    const int lt = it.y;
    const bool vec = d.vec, xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    const float coef = ldf(t.ws + d.bscal);
    const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
    for (int it = 0; it < kFlatIters; ++it) {
        const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
        const int valid = clamp_valid(d.numel - i);
        if (valid == 0) break;
        float x[kVec], m[kVec], v[kVec];
        load_v8(d.x, i, valid, vec, xb, x);
        load_m8(d, i, valid, vec, mb, mi, m);
        load_f8(d.v + i, valid, vec, v);
#pragma unroll
        for (int e = 0; e < kVec; ++e) x[e] = x[e] - coef * lamb_dir(m[e], v[e], x[e], a);
        store_v8(d.x, i, valid, vec, xb, x);
    }
}

void launch_lamb_apply(const Table& t, int64_t n, const LambArgs& a, int storage, hipStream_t s) {
    if (n <= 0) return;
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (storage == kStoreF32) hipLaunchKernelGGL(k_lamb_apply<kStoreF32>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16) hipLaunchKernelGGL(k_lamb_apply<kStoreBf16>, grid, block, 0, s, t, a);
    else if (storage == kStoreF32I8) hipLaunchKernelGGL(k_lamb_apply<kStoreF32I8>, grid, block, 0, s, t, a);
    else if (storage == kStoreBf16I8) hipLaunchKernelGGL(k_lamb_apply<kStoreBf16I8>, grid, block, 0, s, t, a);
    else hipLaunchKernelGGL(k_lamb_apply<kStoreMixed>, grid, block, 0, s, t, a);
}

}  // namespace meo
