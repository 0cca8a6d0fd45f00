// GaLore step: descriptors and launchers shared by galore.hip and the C ABI.
#pragma once
#include "internal.h"

namespace meo {

constexpr int kGaTile = 64;       // rows of the long side per projection tile; short tile side
constexpr int kGaWide = 256;      // long tile side of the back-projection; maximum rank
constexpr int kGaKb = 64;         // contraction block staged in LDS
constexpr int kGaPitch = kGaKb + 8;  // bf16 per LDS row (padding against bank conflicts)
constexpr int kGaProjRB = 1;       // projection tile: 64 kGaProjRB rows of R per block
constexpr int kGaProjRows = kGaTile * kGaProjRB;
constexpr int kGaBackRW = 1;      // back-projection tile: 64 kGaBackRW rows of N per block
constexpr int kGaPwRows = 256;    // wide projection (direct lists): rows of R per block
constexpr int kGaPwThreads = 512; // wide projection: 8 waves

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
    int32_t rvec;       // moment rows ([D][r] fp32) may use 16-byte accesses
    int32_t wvec;       // parameter rows may use 16-byte accesses
    int32_t btj;        // back-projection tiles along the tile's second dimension
};

struct GTable {
    const GDesc* desc;
    const int2* items;  // [grid] x = tensor, y = tile within the tensor; x < 0: an empty
                        // item (padding of the XCD-aligned back-projection list)
};

struct GaArgs {
    float beta1, beta2, omb1, omb2;  // betas and 1 - betas
    float inv_bc1, inv_bc2;          // 1 / (1 - beta^t)
    float eps;
    float decay;                     // 1 - lr * weight_decay
    float coef;                      // lr * scale (projected) or lr (flat)
};

// direct: every tensor of the list has d % kGaKb == 0 and 16-byte rows (vec); the
// list's items are then tiles of kGaPwRows rows of R for the wide kernel, whose
// operands are staged by global_load_lds. Otherwise items are kGaProjRows-row tiles.
void launch_galore_project(const GTable& t, int64_t n, const GaArgs& a, bool left, bool direct, hipStream_t s);
// The wide tiles of both sides in one launch (every tensor of the list direct); the
// items index descriptors of either side, the first nright of them right-side ones.
void launch_galore_project_mixed(const GTable& t, int64_t n, int nright, const GaArgs& a, hipStream_t s);
// Back-projection kernels. kBackReg: operands staged through registers (any list).
// kBackDirect: 64 x 256 tiles staged by global_load_lds (every rank a multiple of kGaKb,
// 16-byte rows). kBackUr / kBackUrBf16: as direct, with U held in registers and items of
// 256 rows of U x up to kUrTiles 64-row tiles of N (item y = band * btj + chunk); every
// parameter of the list fp32 (kBackUr) or bf16 (kBackUrBf16; its m >= n side takes the
// 4-wave, two-blocks-per-CU kernel with 32-row tiles of N over the same items).
enum BackMode { kBackReg = 0, kBackDirect = 1, kBackUr = 2, kBackUrBf16 = 3 };
constexpr int kUrTiles = 64;  // 64-row tiles of N per item of the U-register back-projection
void launch_galore_back(const GTable& t, int64_t n, const GaArgs& a, bool left, int mode, hipStream_t s);
void launch_galore_adamw(const Table& t, int64_t n, const GaArgs& a, hipStream_t s);

// ------------------------------------------------------------------ projector refresh

constexpr int kRfIters = 4;        // subspace iterations per refresh
constexpr int kRfKb = 32;          // contraction block of the refresh products
constexpr int kRfPitch = kRfKb + 8;
constexpr int kRfMaxP = 256;       // iteration block (the rank) at most 256

// One projected tensor of a refresh. X is the gradient oriented so that the
// projector spans its rows' space: X = G (m >= n, D x d) or G^T (m < n). The
// iterate holds p orthonormal rows of length d (the transposed basis).
struct RDesc {
    const uint16_t* g;  // bf16 gradient [m][n]
    uint16_t* u;        // out: projector [d][r], bf16
    uint16_t* ut;       // out: projector transposed [r][d], bf16
    float* qa;          // [p][d] iterate / scratch
    float* qb;          // [p][d] iterate / scratch
    float* yt;          // [p][D] X Q, transposed; later U^T in fp32 [r][d]
    double* s;          // [p][p] Gram matrix, Cholesky factor, eigenproblem
    double* w;          // [p][p] inverse factor, eigenvectors
    double* s2;         // [p][p] second buffer of the eigenproblem
    double* w2;         // [p][p] second buffer of the eigenvectors
    int32_t m, n, D, d, r, p;
    int32_t left;       // m < n
    int32_t gvec;       // gradient rows may use 16-byte loads (n % 8 == 0, aligned)
    int32_t seed;       // index of the tensor in its list (start vectors)
};

struct RTable {
    const RDesc* desc;
    const int2* items;
};

// Buffers named in launches.
enum RBuf { kRbQa = 0, kRbQb = 1, kRbYt = 2 };

void launch_rf_init(const RTable& t, int64_t n, int dst, hipStream_t s);
// out[c][l] = sum_k in[c][k] X?[l][k]: `stage` 0 is Y^T = Q^T X^T (l over D, k over d),
// stage 1 is Z^T = Y^T X (l over d, k over D).
// `trans`: the gradient is read transposed (stage 0 with m < n, stage 1 with m >= n).
void launch_rf_gemm(const RTable& t, int64_t n, int stage, int src, int dst, bool trans, hipStream_t s);
void launch_rf_gram(const RTable& t, int64_t n, int src, bool over_long, hipStream_t s);
void launch_rf_chol(const RTable& t, int64_t n, hipStream_t s);
void launch_rf_trmm(const RTable& t, int64_t n, int src, int dst, hipStream_t s);
void launch_rf_jacobi(const RTable& t, int64_t n, hipStream_t s);
void launch_rf_basis(const RTable& t, int64_t n, int src, hipStream_t s);
void launch_rf_store(const RTable& t, int64_t n, hipStream_t s);

}  // namespace meo
