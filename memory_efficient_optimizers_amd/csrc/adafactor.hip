// Adafactor apply pass: the last streaming pass of the step.
//
// Per element: u = G * rsqrt(C_j) * rsqrt(R_i) * coef_b, where coef_b =
// sqrt(mean R of matrix b) * alpha / kappa (1-D tensors: u = G * rsqrt(V) * coef),
// i.e. the clipped, learning-rate-scaled update of the note after "Step 5" of the
// Colossal-AI distributed-optimizers page. With beta1 (page "Step 3": beta1 set ->
// exp_avg kept) M <- beta1 M + (1 - beta1) u and the step is M; otherwise the step
// is u. The parameter takes decoupled weight decay on its pre-update value:
// X <- X - (weight_decay * alpha) X - step. With 16-bit storage the parameter and
// first moment are widened to fp32 on load and rounded to the nearest bf16 when
// stored; the new first moment is rounded as soon as it is formed, so the step
// is the stored value.
//
// The SQ variant also sums the squares of the updated parameter, as stored, per
// tile: the next step's RMS(X) (scale_parameter) is taken on exactly this
// parameter, so a caller that leaves the parameter alone between steps need not
// read it again for that statistic.
#include "internal.h"

namespace meo {

// 8 fp32 values from two 16-byte words.
__device__ __forceinline__ void f32x8(const u32x4 a, const u32x4 b, float* f) {
    f[0] = __uint_as_float(a.x); f[1] = __uint_as_float(a.y); f[2] = __uint_as_float(a.z); f[3] = __uint_as_float(a.w);
    f[4] = __uint_as_float(b.x); f[5] = __uint_as_float(b.y); f[6] = __uint_as_float(b.z); f[7] = __uint_as_float(b.w);
}

__device__ __forceinline__ u32x4 u4_of(float a, float b, float c, float e) {
    return u32x4{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c), __float_as_uint(e)};
}

__device__ __forceinline__ float sumsq8(const float* f) {
    return ((f[0] * f[0] + f[1] * f[1]) + (f[2] * f[2] + f[3] * f[3])) +
           ((f[4] * f[4] + f[5] * f[5]) + (f[6] * f[6] + f[7] * f[7]));
}

// Sum of the squares of the first `valid` of 8 parameter values as they were
// stored (bf16: rounded to nearest even).
__device__ __forceinline__ float stored_sumsq8(const float* x, int valid, bool bf16) {
    float f[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) f[e] = e < valid ? (bf16 ? round_bf16(x[e]) : x[e]) : 0.0f;
    return sumsq8(f);
}

// The rows of one wave in a 2-D tile with 16-byte aligned rows (W % 8 == 0, so a
// lane has all 8 of its columns or none). The wave's 16 rows are addressed through
// buffer resources: a scalar base per tensor, the row offset in a scalar register
// and one 32-bit lane offset, instead of a 64-bit address per lane and load.
// G16 / S16: gradient / parameter and first moment stored in bf16. RB rows are
// loaded per batch and stay packed until their row is computed; 16-bit storage
// moves half the bytes per row, so it takes twice the rows. W < 2^26 keeps the
// wave's byte range within 32 bits.
template <bool G16, bool S16, bool SQ>
__device__ __forceinline__ float af_rows(const TDesc& d, int lt, float coef, float decay,
                                         const AfApplyArgs& a) {
    constexpr int RB = S16 ? 8 : 4;
    constexpr int GW = G16 ? 1 : 2, SW = S16 ? 1 : 2;       // 16-byte words per lane and row
    constexpr uint32_t GE = G16 ? 2 : 4, SE = S16 ? 2 : 4;  // bytes per element
    const TileRC p = tile_rc(d, lt);
    if (p.valid != kVec || p.nrows <= 0) return 0.0f;
    const bool mom = a.has_beta1;
    float sq = 0.0f;  // sum of the updated X^2 over this lane's rows
    float cf[kVec];
    const float* ccol = d.c + static_cast<int64_t>(p.b) * d.W + p.col;
#pragma unroll
    for (int e = 0; e < kVec; ++e) cf[e] = rsqrtf(ldf(ccol + e));
    const float* rrow = d.r + static_cast<int64_t>(p.b) * d.H + p.row0;
    const int64_t first = (static_cast<int64_t>(p.b) * d.H + p.row0) * d.W;
    const uint32_t n = static_cast<uint32_t>(p.nrows) * static_cast<uint32_t>(d.W);
    const Rsrc rg = make_rsrc(static_cast<const char*>(d.g) + first * GE, n * GE);
    const Rsrc rx = make_rsrc(static_cast<const char*>(d.x) + first * SE, n * SE);
    const Rsrc rm = make_rsrc(mom ? static_cast<const char*>(d.m) + first * SE : nullptr, mom ? n * SE : 0u);
    const uint32_t w = static_cast<uint32_t>(d.W), col = static_cast<uint32_t>(p.col);
    const uint32_t lg = col * GE, ls = col * SE;
    for (int i0 = 0; i0 < p.nrows; i0 += RB) {
        u32x4 gr[RB][GW], xr[RB][SW], mr[RB][SW];
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (i0 + i < p.nrows) {
                const uint32_t r = static_cast<uint32_t>(i0 + i) * w;
#pragma unroll
                for (int k = 0; k < GW; ++k) gr[i][k] = buf_ld(rg, lg + 16u * k, r * GE);
#pragma unroll
                for (int k = 0; k < SW; ++k) xr[i][k] = buf_ld(rx, ls + 16u * k, r * SE);
                if (mom) {
#pragma unroll
                    for (int k = 0; k < SW; ++k) mr[i][k] = buf_ld(rm, ls + 16u * k, r * SE);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            if (i0 + i < p.nrows) {
                const uint32_t r = static_cast<uint32_t>(i0 + i) * w;
                const float rf = rsqrtf(ldf(rrow + i0 + i)) * coef;
                float gf[kVec], xf[kVec], mf[kVec];
                if (G16) bf16x8(gr[i][0], gf); else f32x8(gr[i][0], gr[i][GW - 1], gf);
                if (S16) bf16x8(xr[i][0], xf); else f32x8(xr[i][0], xr[i][SW - 1], xf);
                if (mom) {
                    if (S16) bf16x8(mr[i][0], mf); else f32x8(mr[i][0], mr[i][SW - 1], mf);
                }
                u32x4 mp;
#pragma unroll
                for (int e = 0; e < kVec; e += 2) {
                    float u0 = (gf[e] * cf[e]) * rf, u1 = (gf[e + 1] * cf[e + 1]) * rf;
                    if (mom) {
                        mf[e] = fmaf(a.beta1, mf[e], a.omb1 * u0);
                        mf[e + 1] = fmaf(a.beta1, mf[e + 1], a.omb1 * u1);
                        if (S16) {
                            // rounded once to bf16; the step is the stored value
                            const uint32_t wd = bf16_bits(mf[e]) | (bf16_bits(mf[e + 1]) << 16);
                            mp[e / 2] = wd;
                            mf[e] = bf16_lo(wd);
                            mf[e + 1] = bf16_hi(wd);
                        }
                        u0 = mf[e];
                        u1 = mf[e + 1];
                    }
                    xf[e] = fmaf(-decay, xf[e], xf[e]) - u0;
                    xf[e + 1] = fmaf(-decay, xf[e + 1], xf[e + 1]) - u1;
                }
                if (S16) {
                    if (mom) buf_st(mp, rm, ls, r * SE);
                    const u32x4 xp = pack_bf16x8(xf);
                    buf_st(xp, rx, ls, r * SE);
                    if (SQ) {
                        bf16x8(xp, xf);  // the stored values
                        sq += sumsq8(xf);
                    }
                } else {
                    if (mom) {
                        buf_st(u4_of(mf[0], mf[1], mf[2], mf[3]), rm, ls, r * SE);
                        buf_st(u4_of(mf[4], mf[5], mf[6], mf[7]), rm, ls + 16u, r * SE);
                    }
                    buf_st(u4_of(xf[0], xf[1], xf[2], xf[3]), rx, ls, r * SE);
                    buf_st(u4_of(xf[4], xf[5], xf[6], xf[7]), rx, ls + 16u, r * SE);
                    if (SQ) sq += sumsq8(xf);
                }
            }
        }
    }
    return sq;
}

// One apply tile; returns this thread's sum of the updated X^2 (SQ; else 0), over
// the elements it stored.
template <int ST, bool SQ>
__device__ __forceinline__ float af_tile(const Table& t, const TDesc& d, int lt, const AfApplyArgs& a) {
    const float* ws = t.ws;
    float sq = 0.0f;
    const float decay = ldf(ws + d.scal + kSlotDecay);
    const bool vec = d.vec, bf = d.gbf16, xb = x_is_bf16<ST>(d), mb = m_is_bf16<ST>(d), mi = m_is_i8<ST>(d);
    const bool mom = a.has_beta1;
    const float b1 = a.beta1, omb1 = a.omb1;

    if (d.mode != kFlat) {
        const TileRC p = tile_rc(d, lt);
        const float coef = ldf(ws + d.bscal + p.b);
        if constexpr (ST == kStoreBf16) {
            if (vec && d.W < (1 << 26)) {
                if (bf) return af_rows<true, true, SQ>(d, lt, coef, decay, a);
                return af_rows<false, true, SQ>(d, lt, coef, decay, a);
            }
        }
        const int64_t mat = static_cast<int64_t>(p.b) * d.H * d.W;
        float cf[kVec];
#pragma unroll
        for (int e = 0; e < kVec; ++e)
            cf[e] = e < p.valid ? rsqrtf(ldf(d.c + static_cast<int64_t>(p.b) * d.W + p.col + e)) : 0.0f;
        const float* rrow = d.r + static_cast<int64_t>(p.b) * d.H;
        // Rows per batch: 4 for fp32 storage. 2 for an 8-bit first moment, whose
        // re-quantization needs registers: 90 VGPRs and 5 waves per SIMD instead of
        // 145 and 3, about 10% faster. 2 also for unaligned bf16 rows or mixed
        // storage (rare), which keeps this loop from setting the registers.
        constexpr int RB = ST == kStoreF32 ? 4 : 2;
        for (int i0 = 0; i0 < p.nrows; i0 += RB) {
            float g[RB][kVec], x[RB][kVec], m[RB][kVec];
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i0 + i < p.nrows) {
                    const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                    load_v8(d.g, off, p.valid, vec, bf, g[i]);
                    load_v8(d.x, off, p.valid, vec, xb, x[i]);
                    if (mom) load_m8(d, off, p.valid, vec, mb, mi, m[i]);
                }
            }
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                if (i0 + i < p.nrows) {
                    const int64_t off = mat + static_cast<int64_t>(p.row0 + i0 + i) * d.W + p.col;
                    const float rf = rsqrtf(ldf(rrow + p.row0 + i0 + i)) * coef;
                    float step[kVec];
#pragma unroll
                    for (int e = 0; e < kVec; ++e) step[e] = (g[i][e] * cf[e]) * rf;
                    Q8 q;
                    if (mom) {
#pragma unroll
                        for (int e = 0; e < kVec; ++e) m[i][e] = fmaf(b1, m[i][e], omb1 * step[e]);
                        settle_m8(m[i], mb, mi, q);  // the step is the stored moment
#pragma unroll
                        for (int e = 0; e < kVec; ++e) step[e] = m[i][e];
                    }
#pragma unroll
                    for (int e = 0; e < kVec; ++e) x[i][e] = fmaf(-decay, x[i][e], x[i][e]) - step[e];
                    if (mom) store_m8(d, off, p.valid, vec, mb, mi, m[i], q);
                    store_v8(d.x, off, p.valid, vec, xb, x[i]);
                    if (SQ) sq += stored_sumsq8(x[i], p.valid, xb);
                }
            }
        }
    } else {
        const float coef = ldf(ws + d.bscal);
        const int64_t base = static_cast<int64_t>(lt) * kFlatTile;
        for (int it = 0; it < kFlatIters; ++it) {
            // Block-uniform exit: lanes past the end stay (with nothing to load or
            // store) for the cross-lane work of an 8-bit first moment.
            if (base + static_cast<int64_t>(it) * kThreads * kVec >= d.numel) break;
            const int64_t i = base + (static_cast<int64_t>(it) * kThreads + threadIdx.x) * kVec;
            const int valid = clamp_valid(d.numel - i);
            float g[kVec], v[kVec], x[kVec], m[kVec] = {}, step[kVec];
            load_v8(d.g, i, valid, vec, bf, g);
            load_f8(d.v + i, valid, vec, v);
            load_v8(d.x, i, valid, vec, xb, x);
            if (mom) load_m8(d, i, valid, vec, mb, mi, m);
#pragma unroll
            for (int e = 0; e < kVec; ++e) step[e] = e < valid ? (g[e] * rsqrtf(v[e])) * coef : 0.0f;
            Q8 q;
            if (mom) {
#pragma unroll
                for (int e = 0; e < kVec; ++e) m[e] = fmaf(b1, m[e], omb1 * step[e]);
                settle_m8(m, mb, mi, q);
#pragma unroll
                for (int e = 0; e < kVec; ++e) step[e] = m[e];
            }
#pragma unroll
            for (int e = 0; e < kVec; ++e) x[e] = fmaf(-decay, x[e], x[e]) - step[e];
            if (mom) store_m8(d, i, valid, vec, mb, mi, m, q);
            store_v8(d.x, i, valid, vec, xb, x);
            if (SQ) sq += stored_sumsq8(x, valid, xb);
        }
    }
    return sq;
}

template <int ST, bool SQ>
__global__ __launch_bounds__(kThreads) void k_af_apply(Table t, AfApplyArgs a) {
    const int2 it = t.items[blockIdx.x];
    if (it.x < 0) return;  // an empty item of an XCD-aligned list (the whole block)
    const TDesc d = t.desc[it.x];
    float sq = af_tile<ST, SQ>(t, d, it.y, a);
    if constexpr (SQ) {
        // every thread of the block gets here: af_tile has no barrier and no exit
        // that skips this reduction
        __shared__ float red[2 * kWaves];
        float unused = 0.0f;
        block_sum2(sq, unused, red);
        if (threadIdx.x == 0) stf(t.ws + d.apart + it.y, sq);
    }
}

template <bool SQ>
void launch_af_apply_sq(const Table& t, int64_t n, const AfApplyArgs& a, int storage, hipStream_t s) {
    const dim3 grid(static_cast<uint32_t>(n)), block(kThreads);
    if (storage == kStoreF32) hipLaunchKernelGGL((k_af_apply<kStoreF32, SQ>), grid, block, 0, s, t, a);
    else if (storage == kStoreBf16) hipLaunchKernelGGL((k_af_apply<kStoreBf16, SQ>), grid, block, 0, s, t, a);
    else if (storage == kStoreF32I8) hipLaunchKernelGGL((k_af_apply<kStoreF32I8, SQ>), grid, block, 0, s, t, a);
    else if (storage == kStoreBf16I8) hipLaunchKernelGGL((k_af_apply<kStoreBf16I8, SQ>), grid, block, 0, s, t, a);
    else hipLaunchKernelGGL((k_af_apply<kStoreMixed, SQ>), grid, block, 0, s, t, a);
}

void launch_af_apply(const Table& t, int64_t n, const AfApplyArgs& a, int storage, bool sumsq, hipStream_t s) {
    if (n <= 0) return;
    if (sumsq) launch_af_apply_sq<true>(t, n, a, storage, s);
    else launch_af_apply_sq<false>(t, n, a, storage, s);
}

}  // namespace meo
