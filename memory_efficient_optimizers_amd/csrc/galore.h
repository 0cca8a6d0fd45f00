// GaLore step: descriptors and launchers shared by galore.hip and the C ABI.
#pragma once
#include "internal.h"

namespace meo {

constexpr int kGaTile = 64;       // rows of the long side per projection tile; short tile side
constexpr int kGaWide = 256;      // long tile side of the back-projection; maximum rank
constexpr int kGaKb = 64;         // contraction block staged in LDS
constexpr int kGaPitch = kGaKb + 8;  // bf16 per LDS row (padding against bank conflicts)

// One projected (2-D, bf16-gradient) tensor. With m >= n (right side) the low-rank
// arrays are [m][r] and the projector spans the columns' space (d = n); with m < n
// (left side) they are [n][r] and the projector spans the rows' space (d = m).
struct GDesc {
    const uint16_t* g;  // bf16 gradient [m][n]
    void* x;            // parameter [m][n], fp32 or bf16
    float* em;          // first moment [D][r]
    float* ev;          // second moment [D][r]
    uint16_t* u;        // projector [d][r], bf16
    uint16_t* ut;       // projector transposed [r][d], bf16
    uint16_t* nh;       // workspace: low-rank Adam direction, bf16 high part [D][r]
    uint16_t* nl;       // workspace: bf16 of the remainder [D][r]
    int32_t m, n, D, d, r;
    int32_t xbf16;      // parameter is bf16
    int32_t vec;        // rows of g, u, ut, nh and the moments may use 16-byte accesses
    int32_t btj;        // back-projection tiles along the tile's second dimension
};

struct GTable {
    const GDesc* desc;
    const int2* items;  // [grid] x = tensor, y = tile within the tensor
};

struct GaArgs {
    float beta1, beta2, omb1, omb2;  // betas and 1 - betas
    float inv_bc1, inv_bc2;          // 1 / (1 - beta^t)
    float eps;
    float decay;                     // 1 - lr * weight_decay
    float coef;                      // lr * scale (projected) or lr (flat)
};

void launch_galore_project(const GTable& t, int64_t n, const GaArgs& a, bool left, hipStream_t s);
void launch_galore_back(const GTable& t, int64_t n, const GaArgs& a, bool left, hipStream_t s);
void launch_galore_adamw(const Table& t, int64_t n, const GaArgs& a, hipStream_t s);

}  // namespace meo
