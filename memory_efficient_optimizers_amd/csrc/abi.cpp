// C ABI of the optimizer-step library: validation, launch tables, pass sequences.
//
// Host-side schedule values are computed in fp64 from the rules on the
// Colossal-AI distributed-optimizers page: the relative step size
// min(1e-2, 1/sqrt(step)) (1e-6*step with warmup_init) and its errors from
// section "Step 3", beta2t = 1 - step**decay_rate from the note after "Step 5";
// CAME and LAMB defaults and checks from the DistributedCAME / DistributedLAMB
// paragraphs. Everything per element runs in the HIP passes.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <list>
#include <mutex>
#include <string>
#include <vector>

#include "meo.h"
#include "internal.h"
#include "galore.h"

using namespace meo;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

enum Op { kOpAdafactor = 0, kOpCame = 1, kOpLamb = 2 };

void release_galore_plans();  // GaLore launch tables (defined with the GaLore entry points)

uintptr_t elem_bytes(int32_t dtype) { return dtype == MEO_F32 ? 4 : (dtype == MEO_BF16 ? 2 : 1); }

// Uniform view of the per-tensor state pointers of the three optimizers.
struct StatePtrs {
    void* m = nullptr;   // float32, bf16 or int8 codes (the tensor's state_dtype)
    float* ms = nullptr; // scales of an 8-bit first moment
    float* v = nullptr;
    float* r = nullptr;
    float* c = nullptr;
    float* rr = nullptr;
    float* rc = nullptr;
    float* xsq = nullptr; // Adafactor: carried sum(X^2) [1]
};

constexpr int64_t kMaxDim = (int64_t{1} << 31) - 1;

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t align64(int64_t f) { return (f + 63) / 64 * 64; }  // floats -> 256-byte multiple

bool is_factored(int op, const meo_tensor& t) { return op != kOpLamb && t.ndim >= 2; }

bool overflow_numel(const meo_tensor& t, int64_t* numel) {
    __int128 n = static_cast<__int128>(t.batch) * t.rows * t.cols;
    if (n > (static_cast<__int128>(1) << 62)) return true;
    *numel = static_cast<int64_t>(n);
    return false;
}

// Geometry and workspace layout of one tensor. It depends on the shapes and on the
// alignment of param and grad (which decides the statistics mode), not on states.
struct Geo {
    int64_t numel = 0;
    int32_t mode = kFlat, cls = 0, B = 1, H = 1, W = 1, tr = 1, tc = 0, strips = 0, srows = 0, nrc = 0, ncc = 0;
    int64_t tiles = 0;  // 2-D tiles (factored) or flat tiles
    int32_t xchunks = 0;
    int64_t rowpart = 0, colpart = 0, sumr = 0, tilepart = 0, xpart = 0, apart = 0, bscal = 0, scal = 0;
};

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Adafactor's strip height for rows wider than 4096 (the second row-complete
// class): their few strips per matrix (an 11008-wide, 4096-row matrix makes 32 of
// 128 rows) leave the GPU underfilled on small lists. Measured side by side, 64
// rows take one Llama layer's step 5% lower and the 7B list's 0.2% higher (more
// column partials).
constexpr int kStripRowsWide = 64;

// Fills geometry and workspace offsets; returns the workspace size in floats.
// Tensors are assumed validated.
int64_t layout(int op, int32_t n, const meo_tensor* ts, std::vector<Geo>* out) {
    int64_t off = 0;
    if (out) out->assign(n, Geo());
    for (int32_t k = 0; k < n; ++k) {
        Geo g;
        overflow_numel(ts[k], &g.numel);
        if (g.numel > 0) {
            if (is_factored(op, ts[k])) {
                g.B = static_cast<int32_t>(ts[k].batch);
                g.H = static_cast<int32_t>(ts[k].rows);
                g.W = static_cast<int32_t>(ts[k].cols);
                const bool rc_ok = g.W % kVec == 0 && g.W <= kRcMaxCols1 && aligned16(ts[k].param) &&
                                   aligned16(ts[k].grad);
                g.mode = rc_ok ? kRowComplete : kTiled;
                g.cls = g.W <= kRcMaxCols0 ? 0 : 1;
                g.tr = static_cast<int32_t>(ceil_div(g.H, kTileRows));
                g.tc = static_cast<int32_t>(ceil_div(g.W, kTileCols));
                g.srows = op != kOpAdafactor ? kStripRowsCame : (g.cls == 0 ? kStripRowsAdafactor : kStripRowsWide);
                g.strips = static_cast<int32_t>(ceil_div(g.H, g.srows));
                g.tiles = static_cast<int64_t>(g.B) * g.tr * g.tc;
                g.nrc = static_cast<int32_t>(ceil_div(g.H, kFinChunk));
                g.ncc = static_cast<int32_t>(ceil_div(g.W, kFinCols));
                const bool tiled_stats = g.mode == kTiled || op == kOpCame;  // CAME's confidence is tiled
                const int64_t B = g.B;
                const int64_t colrows = std::max<int64_t>(tiled_stats ? g.tr : 0,
                                                          g.mode == kRowComplete ? 2 * int64_t{g.strips} : 0);
                const int64_t tparts = std::max<int64_t>(g.mode == kTiled ? g.tiles : 0,
                                                         g.mode == kRowComplete ? B * g.strips : 0);
                g.rowpart = off; off = align64(off + (tiled_stats ? B * g.tc * g.H : 0));
                g.colpart = off; off = align64(off + B * colrows * g.W);
                g.sumr = off;    off = align64(off + B * std::max(g.nrc, g.ncc));
                g.tilepart = off; off = align64(off + 2 * tparts);
                if (g.mode == kRowComplete) {
                    g.xchunks = static_cast<int32_t>(ceil_div(g.numel, kFlatTile));
                    g.xpart = off; off = align64(off + g.xchunks);
                }
            } else {
                g.mode = kFlat;
                g.tiles = ceil_div(g.numel, kFlatTile);
                g.tc = static_cast<int32_t>(g.tiles);
                g.tilepart = off; off = align64(off + 2 * g.tiles);
            }
            if (op == kOpAdafactor) {  // the apply pass's sums of the updated X^2
                g.apart = off; off = align64(off + g.tiles);
            }
            g.bscal = off; off = align64(off + 2 * static_cast<int64_t>(g.B));
            g.scal = off;  off = align64(off + kScalSlots);
        }
        if (out) (*out)[k] = g;
    }
    return off;
}

// ----------------------------------------------------------------------------- validation

bool finite(double v) { return std::isfinite(v); }

// The first moment of tensor k, when the step uses it: present and aligned for
// its dtype; an 8-bit one also needs its scales and, for a factored tensor,
// cols % 128 == 0 (no quantization group crosses a row).
int check_moment(int op, int32_t k, const meo_tensor& t, const void* m, const float* scale, const char* why) {
    int64_t numel = 0;
    overflow_numel(t, &numel);
    if (numel == 0) return MEO_OK;
    const std::string who = "tensor " + std::to_string(k) + ": ";
    if (!m) return fail(MEO_ENULL, who + "exp_avg is NULL" + why);
    if (reinterpret_cast<uintptr_t>(m) % elem_bytes(t.state_dtype)) return fail(MEO_EALIGN, who + "exp_avg misaligned");
    if (t.state_dtype == MEO_I8) {
        if (!scale) return fail(MEO_ENULL, who + "exp_avg_scale is NULL (8-bit first moment)");
        if (reinterpret_cast<uintptr_t>(scale) % 4) return fail(MEO_EALIGN, who + "exp_avg_scale misaligned");
        if (is_factored(op, t) && t.cols % kI8Group != 0)
            return fail(MEO_ESHAPE, who + "an 8-bit first moment of a factored tensor needs cols % 128 == 0");
    }
    return MEO_OK;
}

int check_tensors(int op, int64_t step, int32_t n, const meo_tensor* ts, const void* states) {
    if (step < 1) return fail(MEO_EINVAL, "step must be >= 1 (1-based index of the step being taken)");
    if (n < 0) return fail(MEO_EINVAL, "negative tensor count");
    if (n == 0) return MEO_OK;
    if (!ts) return fail(MEO_ENULL, "tensors is NULL");
    if (!states) return fail(MEO_ENULL, "states is NULL");
    int64_t total_tiles = 0, total_fin = 0;
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        const std::string who = "tensor " + std::to_string(k) + ": ";
        if (t.batch < 0 || t.rows < 0 || t.cols < 0 || t.ndim < 0)
            return fail(MEO_ESHAPE, who + "negative batch, rows, cols or ndim");
        int64_t numel;
        if (overflow_numel(t, &numel)) return fail(MEO_ESHAPE, who + "too many elements");
        if (t.ndim <= 1 && numel > 0 && (t.batch != 1 || t.rows != 1))
            return fail(MEO_ESHAPE, who + "a tensor with ndim <= 1 must have batch == rows == 1");
        if (t.param_dtype != MEO_F32 && t.param_dtype != MEO_BF16)
            return fail(MEO_EDTYPE, who + "param_dtype must be MEO_F32 or MEO_BF16");
        if (t.grad_dtype != MEO_F32 && t.grad_dtype != MEO_BF16)
            return fail(MEO_EDTYPE, who + "grad_dtype must be MEO_F32 or MEO_BF16");
        if (t.state_dtype != MEO_F32 && t.state_dtype != MEO_BF16 && t.state_dtype != MEO_I8)
            return fail(MEO_EDTYPE, who + "state_dtype must be MEO_F32, MEO_BF16 or MEO_I8");
        if (numel == 0) continue;
        if (!t.param) return fail(MEO_ENULL, who + "param is NULL");
        if (!t.grad) return fail(MEO_ENULL, who + "grad is NULL");
        if (reinterpret_cast<uintptr_t>(t.param) % (t.param_dtype == MEO_BF16 ? 2 : 4))
            return fail(MEO_EALIGN, who + "param misaligned for its dtype");
        if (reinterpret_cast<uintptr_t>(t.grad) % (t.grad_dtype == MEO_BF16 ? 2 : 4))
            return fail(MEO_EALIGN, who + "grad misaligned for its dtype");
        const bool fac = is_factored(op, t);
        if (fac) {
            if (t.batch > kMaxDim || t.rows > kMaxDim || t.cols > kMaxDim)
                return fail(MEO_ESHAPE, who + "batch, rows or cols exceed 2^31 - 1");
            const int64_t tiles = t.batch * ceil_div(t.rows, kTileRows) * ceil_div(t.cols, kTileCols);
            if (tiles > kMaxDim) return fail(MEO_ESHAPE, who + "too many tiles");
            total_tiles += tiles;
            total_fin += t.batch * (ceil_div(t.rows, kFinChunk) + ceil_div(t.cols, kFinCols));
        } else {
            total_tiles += ceil_div(numel, kFlatTile);
        }
        // states
        StatePtrs sp;
        if (op == kOpAdafactor) {
            const auto& s = static_cast<const meo_adafactor_state*>(states)[k];
            sp.m = s.exp_avg; sp.r = s.exp_avg_sq_row; sp.c = s.exp_avg_sq_col; sp.v = s.exp_avg_sq;
            sp.ms = s.exp_avg_scale;
        } else if (op == kOpCame) {
            const auto& s = static_cast<const meo_came_state*>(states)[k];
            sp.m = s.exp_avg; sp.r = s.exp_avg_sq_row; sp.c = s.exp_avg_sq_col; sp.ms = s.exp_avg_scale;
            sp.rr = s.exp_avg_res_row; sp.rc = s.exp_avg_res_col; sp.v = s.exp_avg_sq;
        } else {
            const auto& s = static_cast<const meo_lamb_state*>(states)[k];
            sp.m = s.exp_avg; sp.v = s.exp_avg_sq; sp.ms = s.exp_avg_scale;
        }
        const void* need[6] = {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr};
        const char* names[6] = {"", "", "", "", "", ""};
        uintptr_t align[6] = {4, 4, 4, 4, 4, 4};
        int nn = 0;
        if (op == kOpLamb) {
            align[nn] = elem_bytes(t.state_dtype);
            need[nn] = sp.m; names[nn++] = "exp_avg";
            need[nn] = sp.v; names[nn++] = "exp_avg_sq";
        } else {
            if (fac) {
                need[nn] = sp.r; names[nn++] = "exp_avg_sq_row";
                need[nn] = sp.c; names[nn++] = "exp_avg_sq_col";
                if (op == kOpCame) {
                    need[nn] = sp.rr; names[nn++] = "exp_avg_res_row";
                    need[nn] = sp.rc; names[nn++] = "exp_avg_res_col";
                }
            } else {
                need[nn] = sp.v; names[nn++] = "exp_avg_sq";
            }
        }
        for (int i = 0; i < nn; ++i) {
            if (!need[i]) return fail(MEO_ENULL, who + names[i] + " is NULL");
            if (reinterpret_cast<uintptr_t>(need[i]) % align[i])
                return fail(MEO_EALIGN, who + names[i] + " misaligned");
        }
    }
    if (total_tiles > 0xffffffffLL || total_fin > 0xffffffffLL)
        return fail(MEO_ESHAPE, "the tensor list needs more than 2^32 blocks in one pass");
    return MEO_OK;
}

int check_adafactor_hp(const meo_adafactor_hparams* hp) {
    if (!hp) return fail(MEO_ENULL, "hparams is NULL");
    if (hp->has_lr && hp->relative_step)
        return fail(MEO_EINVAL, "Cannot combine manual lr and relative_step=True options");
    if (hp->warmup_init && !hp->relative_step)
        return fail(MEO_EINVAL, "warmup_init=True requires relative_step=True");
    if (!hp->has_lr && !hp->relative_step) return fail(MEO_EINVAL, "lr is required when relative_step=False");
    if (hp->has_lr && !(finite(hp->lr) && hp->lr >= 0.0)) return fail(MEO_EINVAL, "Invalid learning rate");
    if (!(finite(hp->eps1) && hp->eps1 >= 0.0 && finite(hp->eps2) && hp->eps2 >= 0.0))
        return fail(MEO_EINVAL, "eps must be finite and >= 0");
    if (!(finite(hp->clip_threshold) && hp->clip_threshold > 0.0))
        return fail(MEO_EINVAL, "clip_threshold must be finite and > 0");
    if (!finite(hp->decay_rate)) return fail(MEO_EINVAL, "decay_rate must be finite");
    if (hp->has_beta1 && !finite(hp->beta1)) return fail(MEO_EINVAL, "beta1 must be finite");
    if (!finite(hp->weight_decay)) return fail(MEO_EINVAL, "weight_decay must be finite");
    return MEO_OK;
}

int check_came_hp(const meo_came_hparams* hp) {
    if (!hp) return fail(MEO_ENULL, "hparams is NULL");
    if (!hp->has_lr) return fail(MEO_EINVAL, "CAME requires an explicit lr");
    if (!(finite(hp->lr) && hp->lr >= 0.0)) return fail(MEO_EINVAL, "Invalid learning rate");
    const double b[3] = {hp->beta1, hp->beta2, hp->beta3};
    for (int i = 0; i < 3; ++i)
        if (!(b[i] >= 0.0 && b[i] < 1.0))
            return fail(MEO_EINVAL, "Invalid beta parameter at index " + std::to_string(i));
    if (!(finite(hp->eps1) && hp->eps1 >= 0.0 && finite(hp->eps2) && hp->eps2 >= 0.0))
        return fail(MEO_EINVAL, "eps must be finite and >= 0");
    if (!(finite(hp->clip_threshold) && hp->clip_threshold > 0.0))
        return fail(MEO_EINVAL, "clip_threshold must be finite and > 0");
    if (!finite(hp->weight_decay)) return fail(MEO_EINVAL, "weight_decay must be finite");
    return MEO_OK;
}

int check_lamb_hp(const meo_lamb_hparams* hp) {
    if (!hp) return fail(MEO_ENULL, "hparams is NULL");
    if (!(finite(hp->lr) && hp->lr >= 0.0)) return fail(MEO_EINVAL, "Invalid learning rate");
    if (!(finite(hp->eps) && hp->eps >= 0.0)) return fail(MEO_EINVAL, "Invalid epsilon value");
    if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0)) return fail(MEO_EINVAL, "Invalid beta parameter at index 0");
    if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0)) return fail(MEO_EINVAL, "Invalid beta parameter at index 1");
    if (!finite(hp->weight_decay)) return fail(MEO_EINVAL, "weight_decay must be finite");
    return MEO_OK;
}

// Offsets (floats) of each tensor's record of partial sums in a row-sharded step,
// and the total; the layout is the one meo.h documents.
int64_t partials_layout(int op, int32_t n, const meo_tensor* ts, std::vector<int64_t>* offs) {
    int64_t off = 0;
    if (offs) offs->assign(n, 0);
    for (int32_t k = 0; k < n; ++k) {
        int64_t numel = 0;
        overflow_numel(ts[k], &numel);
        if (offs) (*offs)[k] = off;
        // Every tensor has its record, also where this rank holds none of it, so that
        // the ranks' buffers line up for the all-reduce.
        if (is_factored(op, ts[k])) off += ts[k].batch * (2 * ts[k].cols + 1) + 1;
        else off += 2;
    }
    return off;
}

// CAME's second record (confidence sums): [B][W] + [B] per factored tensor, none for
// 1-D tensors (their step ends in the moment pass).
int64_t confidence_layout(int32_t n, const meo_tensor* ts, std::vector<int64_t>* offs) {
    int64_t off = 0;
    if (offs) offs->assign(n, 0);
    for (int32_t k = 0; k < n; ++k) {
        if (offs) (*offs)[k] = off;
        if (is_factored(kOpCame, ts[k])) off += ts[k].batch * (ts[k].cols + 1);
    }
    return off;
}

// Whether [p, p + bytes) lies in one allocation of device memory of device `dev`
// that the HIP runtime knows (hipMalloc, hipMallocManaged, allocators built on
// them). Catches host, truncated or stale pointers and ranges described past the
// end of their memory before any kernel touches them. Returns `code` on failure.
int check_device_range(const void* p, size_t bytes, int dev, const std::string& what, int code) {
    hipPointerAttribute_t attr;
    if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
        (void)hipGetLastError();
        return fail(code, what + " is not device memory known to HIP");
    }
    if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
        return fail(code, what + " is not device memory");
    if (attr.type == hipMemoryTypeDevice && attr.device != dev)
        return fail(code, what + " is on device " + std::to_string(attr.device) + ", the current device is " +
                              std::to_string(dev));
    void* base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return fail(code, what + ": the extent of its allocation is unknown to HIP");
    }
    const uintptr_t b = reinterpret_cast<uintptr_t>(base), q = reinterpret_cast<uintptr_t>(p);
    if (q < b || bytes > size - (q - b))
        return fail(code, what + " (" + std::to_string(bytes) + " bytes) extends past the end of its allocation");
    return MEO_OK;
}

int check_workspace(int op, int32_t n, const meo_tensor* ts, void* ws, size_t bytes) {
    const int64_t need = layout(op, n, ts, nullptr) * static_cast<int64_t>(sizeof(float));
    if (need == 0) return MEO_OK;
    if (!ws) return fail(MEO_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MEO_EWORKSPACE, "workspace not 256-byte aligned");
    if (bytes < static_cast<size_t>(need))
        return fail(MEO_EWORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MEO_EHIP, "hipGetDevice failed");
    }
    return check_device_range(ws, bytes, dev, "workspace", MEO_EWORKSPACE);
}

// Every pointer of the list against its allocation (at launch-table creation; a
// cached table stands for pointers that were checked).
int check_tensor_memory(int op, int32_t n, const meo_tensor* ts, const StatePtrs* sp, int has_m, int dev) {
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        int64_t numel = 0;
        overflow_numel(t, &numel);
        if (numel == 0) continue;
        const std::string who = "tensor " + std::to_string(k) + ": ";
        const size_t ne = static_cast<size_t>(numel);
        const size_t rows = static_cast<size_t>(t.batch * t.rows), cols = static_cast<size_t>(t.batch * t.cols);
        struct Range { const void* p; size_t bytes; const char* name; };
        std::vector<Range> rs = {{t.param, ne * (t.param_dtype == MEO_BF16 ? 2 : 4), "param"},
                                 {t.grad, ne * (t.grad_dtype == MEO_BF16 ? 2 : 4), "grad"}};
        if (has_m) rs.push_back({sp[k].m, ne * elem_bytes(t.state_dtype), "exp_avg"});
        if (has_m && t.state_dtype == MEO_I8)
            rs.push_back({sp[k].ms, static_cast<size_t>((numel + kI8Group - 1) / kI8Group) * 4, "exp_avg_scale"});
        if (is_factored(op, t)) {
            rs.push_back({sp[k].r, rows * 4, "exp_avg_sq_row"});
            rs.push_back({sp[k].c, cols * 4, "exp_avg_sq_col"});
            if (op == kOpCame) {
                rs.push_back({sp[k].rr, rows * 4, "exp_avg_res_row"});
                rs.push_back({sp[k].rc, cols * 4, "exp_avg_res_col"});
            }
        } else {
            rs.push_back({sp[k].v, ne * 4, "exp_avg_sq"});
        }
        if (sp[k].xsq) rs.push_back({sp[k].xsq, 4, "param_sumsq"});
        for (const Range& r : rs) {
            const int rc = check_device_range(r.p, r.bytes, dev, who + r.name, MEO_EMEMORY);
            if (rc) return rc;
        }
    }
    return MEO_OK;
}

// Offsets (floats) of each tensor's scalar slots in the workspace, -1 for tensors
// with zero elements; the layout the step calls use for the same list.
int scalar_offsets(int op, int32_t n, const meo_tensor* ts, int64_t* out) {
    g_err.clear();
    if (n < 0) return fail(MEO_ESHAPE, "n must be >= 0");
    if (n == 0) return MEO_OK;
    if (!ts || !out) return fail(MEO_ENULL, "tensors and offsets must not be NULL");
    for (int32_t k = 0; k < n; ++k) {
        int64_t numel = 0;
        if (ts[k].batch < 0 || ts[k].rows < 0 || ts[k].cols < 0 || overflow_numel(ts[k], &numel) ||
            (is_factored(op, ts[k]) && (ts[k].batch > kMaxDim || ts[k].rows > kMaxDim || ts[k].cols > kMaxDim)))
            return fail(MEO_ESHAPE, "tensor " + std::to_string(k) + ": invalid batch/rows/cols");
    }
    std::vector<Geo> geo;
    layout(op, n, ts, &geo);
    for (int32_t k = 0; k < n; ++k) out[k] = geo[k].numel > 0 ? geo[k].scal : -1;
    return MEO_OK;
}

// ----------------------------------------------------------------------------- plan cache

// Item tables of the launches of one call.
enum List { kListRc0 = 0, kListRc1, kListTiled, kListAll, kListFin1, kListFin2, kListShard, kListFold, kListEmpty,
            kListConfRows, kListConf, kListEmpty2, kListXnorm, kListCameApply, kListCount };

struct Plan {
    std::vector<uint8_t> key;
    int device = 0;
    void* mem = nullptr;  // [n TDesc][item tables]
    int32_t n = 0;
    int32_t storage = kStoreF32;  // Storage class of the list's parameters and first moments
    const TDesc* desc = nullptr;
    const int2* items[kListCount] = {};
    int64_t count[kListCount] = {};
};

std::mutex g_mu;
std::list<Plan*> g_plans;  // most recently used first
// Cached lists per kind (whole-tensor / row-sharded steps, GaLore). Evicting one frees
// its device memory, which waits for the device.
constexpr size_t kMaxPlans = 64;

void free_plan(Plan* p) {
    int cur = 0;
    (void)hipGetDevice(&cur);
    if (cur != p->device) (void)hipSetDevice(p->device);
    (void)hipFree(p->mem);  // waits for work still using it
    if (cur != p->device) (void)hipSetDevice(cur);
    delete p;
}

// One parameter type for the whole list, and one first-moment type among the
// tensors that keep a moment: fp32/fp32, bf16/bf16, fp32/int8 or bf16/int8;
// anything else is mixed (types read per tensor).
int32_t storage_class(const std::vector<TDesc>& desc) {
    if (desc.empty()) return kStoreF32;
    const bool xb = desc[0].xbf16 != 0;
    int mkind = -1;  // 0 fp32, 1 bf16, 2 int8; -1 no moment seen
    for (const TDesc& d : desc) {
        if ((d.xbf16 != 0) != xb) return kStoreMixed;
        if (!d.m) continue;
        const int k = d.mi8 ? 2 : (d.mbf16 ? 1 : 0);
        if (mkind >= 0 && k != mkind) return kStoreMixed;
        mkind = k;
    }
    if (mkind == 2) return xb ? kStoreBf16I8 : kStoreF32I8;
    if (mkind == -1) return xb ? kStoreBf16 : kStoreF32;
    if (mkind == (xb ? 1 : 0)) return xb ? kStoreBf16 : kStoreF32;
    return kStoreMixed;
}

// Reorders a streaming list so that all column tiles of one row tile (a factored
// tensor's tiles that share rows) run on the same XCD. Blocks are dispatched to the
// 8 XCDs round-robin by block index, so the row tiles are dealt to 8 queues and the
// queues are interleaved; where a queue runs out, an empty item (x = -1, the block
// returns at once) keeps the others aligned. This lets one L2 gather the partial
// writes of a row's 8-bit scales (128 values per 4-byte scale, 16 bytes per
// 512-column tile) into whole lines. Results do not depend on the order.
constexpr int kXcds = 8;
void xcd_order(std::vector<int2>& items, const std::vector<TDesc>& desc) {
    std::vector<std::vector<int2>> q(kXcds);
    size_t i = 0, run = 0;
    while (i < items.size()) {
        const TDesc& d = desc[items[i].x];
        const size_t per = d.mode == kFlat ? 1 : static_cast<size_t>(d.tc);  // items of one row tile
        const size_t j = std::min(items.size(), i + per);
        for (size_t k = i; k < j; ++k) q[run % kXcds].push_back(items[k]);
        ++run;
        i = j;
    }
    size_t longest = 0;
    for (const auto& v : q) longest = std::max(longest, v.size());
    std::vector<int2> out;
    out.reserve(longest * kXcds);
    for (size_t r = 0; r < longest; ++r)
        for (int x = 0; x < kXcds; ++x) out.push_back(r < q[x].size() ? q[x][r] : make_int2(-1, -1));
    items.swap(out);
}

// The key of a list's launch tables: everything they are built from.
std::vector<uint8_t> plan_key(int op, int32_t n, const meo_tensor* ts, const StatePtrs* sp, int has_m, int dev,
                              const meo_shard* shards) {
    const size_t nsh = shards ? n * sizeof(meo_shard) : 0;
    std::vector<uint8_t> key(sizeof(int) * 5 + n * (sizeof(meo_tensor) + sizeof(StatePtrs)) + nsh);
    uint8_t* w = key.data();
    const int hdr[5] = {op, n, dev, has_m, shards ? 1 : 0};
    std::memcpy(w, hdr, sizeof hdr); w += sizeof hdr;
    std::memcpy(w, ts, n * sizeof(meo_tensor)); w += n * sizeof(meo_tensor);
    std::memcpy(w, sp, n * sizeof(StatePtrs)); w += n * sizeof(StatePtrs);
    if (nsh) std::memcpy(w, shards, nsh);
    return key;
}

// The launch tables of one list in host memory: [n TDesc][item tables], each
// table 256-byte aligned at offs[l] with count[l] items.
struct HostPlan {
    std::vector<uint8_t> bytes;
    size_t offs[kListCount] = {};
    int64_t count[kListCount] = {};
    int32_t n = 0;
    int32_t storage = kStoreF32;
};

// Deals whole tensors (runs of items with one tensor index) to the 8 XCD queues,
// largest first onto the least loaded queue, then interleaves the queues so that
// block i runs on XCD i % 8: every tile of a tensor runs on one XCD, whose L2
// then fetches that tensor's shared operands once. Empty items (x = -1) pad the
// shorter queues.
void xcd_deal(std::vector<int2>& items) {
    std::vector<std::pair<size_t, size_t>> runs;
    for (size_t i = 0; i < items.size();) {
        size_t j = i;
        while (j < items.size() && items[j].x == items[i].x) ++j;
        if (items[i].x >= 0) runs.push_back({i, j});
        i = j;
    }
    std::vector<size_t> order(runs.size());
    for (size_t i = 0; i < order.size(); ++i) order[i] = i;
    std::stable_sort(order.begin(), order.end(), [&](size_t a, size_t b) {
        return runs[a].second - runs[a].first > runs[b].second - runs[b].first;
    });
    std::vector<std::vector<int2>> q(kXcds);
    for (size_t r : order) {
        size_t best = 0;
        for (size_t x = 1; x < q.size(); ++x)
            if (q[x].size() < q[best].size()) best = x;
        q[best].insert(q[best].end(), items.begin() + runs[r].first, items.begin() + runs[r].second);
    }
    size_t longest = 0;
    for (const auto& v : q) longest = std::max(longest, v.size());
    std::vector<int2> out;
    out.reserve(longest * kXcds);
    for (size_t r = 0; r < longest; ++r)
        for (int x = 0; x < kXcds; ++x) out.push_back(r < q[x].size() ? q[x][r] : make_int2(-1, -1));
    items.swap(out);
}

// Builds the launch tables of a list on the host (no device memory is touched or
// allocated); first checks every pointer of the list against its allocation.
// `shards` (row-sharded steps; else null): the whole tensors' sizes.
int build_host_plan(int op, int32_t n, const meo_tensor* ts, const StatePtrs* sp, int has_m, int dev,
                    const meo_shard* shards, HostPlan* out) {
    int rc = check_tensor_memory(op, n, ts, sp, has_m, dev);
    if (rc) return rc;
    std::vector<Geo> geo;
    layout(op, n, ts, &geo);
    std::vector<int64_t> poff, poff2;
    if (shards) partials_layout(op, n, ts, &poff);
    if (shards && op == kOpCame) confidence_layout(n, ts, &poff2);
    std::vector<TDesc> desc;
    std::vector<int2> lists[kListCount];
    for (int32_t k = 0; k < n; ++k) {
        const Geo& g = geo[k];
        if (g.numel == 0) {
            if (shards) {  // a rank with none of the tensor contributes zeros
                const int64_t len = (k + 1 < n ? poff[k + 1] : partials_layout(op, n, ts, nullptr)) - poff[k];
                lists[kListEmpty].push_back(make_int2(static_cast<int>(poff[k]), static_cast<int>(len)));
                if (op == kOpCame) {
                    const int64_t len2 = (k + 1 < n ? poff2[k + 1] : confidence_layout(n, ts, nullptr)) - poff2[k];
                    if (len2 > 0)
                        lists[kListEmpty2].push_back(make_int2(static_cast<int>(poff2[k]), static_cast<int>(len2)));
                }
            }
            continue;
        }
        const int32_t id = static_cast<int32_t>(desc.size());
        TDesc d;
        std::memset(&d, 0, sizeof d);
        d.x = ts[k].param;
        d.g = ts[k].grad;
        d.m = has_m ? sp[k].m : nullptr;
        d.v = sp[k].v; d.r = sp[k].r; d.c = sp[k].c; d.rr = sp[k].rr; d.rc = sp[k].rc;
        d.numel = g.numel;
        d.rowpart = g.rowpart; d.colpart = g.colpart; d.sumr = g.sumr;
        d.tilepart = g.tilepart; d.xpart = g.xpart; d.apart = g.apart; d.bscal = g.bscal; d.scal = g.scal;
        d.xsq = sp[k].xsq;
        d.xchunks = g.xchunks;
        d.B = g.B; d.H = g.H; d.W = g.W;
        d.mode = g.mode;
        d.gbf16 = ts[k].grad_dtype == MEO_BF16;
        d.xbf16 = ts[k].param_dtype == MEO_BF16;
        d.mbf16 = ts[k].state_dtype == MEO_BF16;
        d.mi8 = has_m && ts[k].state_dtype == MEO_I8;
        d.ms = d.mi8 ? sp[k].ms : nullptr;
        bool vec = aligned16(d.x) && aligned16(d.g) && (!d.m || aligned16(d.m));
        if (g.mode != kFlat) vec = vec && (g.W % kVec == 0);
        else vec = vec && (!d.v || aligned16(d.v));
        d.vec = vec;
        d.tr = g.tr; d.tc = g.tc; d.strips = g.strips; d.srows = g.srows;
        d.nrc = g.nrc; d.ncc = g.ncc;
        if (shards) {
            d.part = poff[k];
            d.total = shards[k].rows_total;
            if (op == kOpCame) d.part2 = poff2[k];
        }
        desc.push_back(d);
        auto add = [&](int list, int64_t count) {
            for (int64_t i = 0; i < count; ++i) lists[list].push_back(make_int2(id, static_cast<int>(i)));
        };
        if (shards) {  // the record of partial sums, and (factored) its fold
            const int64_t per = g.mode == kFlat ? 1 : static_cast<int64_t>(g.B) * ceil_div(g.W, kThreads);
            add(kListShard, per);
            if (g.mode != kFlat) add(kListFold, per);
            if (op == kOpCame && g.mode != kFlat) {
                add(kListConf, per);
                // the row items of the confidence finalize (its tiled layout: nrc row
                // chunks then ncc column chunks per matrix)
                for (int32_t b = 0; b < g.B; ++b)
                    for (int32_t j = 0; j < g.nrc; ++j)
                        lists[kListConfRows].push_back(make_int2(id, b * (g.nrc + g.ncc) + j));
            }
        }
        if (g.mode == kFlat) {
            add(kListAll, g.tiles);
            if (op != kOpLamb) add(kListRc0, g.tiles);
        } else {
            add(kListAll, g.tiles);
            if (g.mode == kRowComplete) {
                add(g.cls == 0 ? kListRc0 : kListRc1, static_cast<int64_t>(g.B) * g.strips);
                if (op == kOpAdafactor) add(kListXnorm, g.xchunks);  // only Adafactor uses RMS(X)
                add(kListFin1, static_cast<int64_t>(g.B) * g.ncc);
            } else {
                add(kListTiled, g.tiles);
                add(kListFin1, static_cast<int64_t>(g.B) * (g.nrc + g.ncc));
            }
            if (op == kOpCame) {
                add(kListFin2, static_cast<int64_t>(g.B) * (g.nrc + g.ncc));
                // the apply: kFlatTile-element ranges in memory order where the rows
                // are 16-byte aligned, 64 x 512 tiles otherwise
                add(kListCameApply, vec ? ceil_div(static_cast<int64_t>(g.B) * g.H * g.W, kFlatTile) : g.tiles);
            }
        }
    }
    // Measured in-process: 3% faster steps with 8-bit first moments, no gain (or a
    // 1% loss with bf16 storage) where no line is shared between tiles; CAME's moment
    // pass (the only CAME launch over kListAll in a whole step) 1% faster over the
    // Llama-7B list and unchanged over one layer.
    bool any_i8 = false;
    for (const TDesc& d : desc) any_i8 = any_i8 || d.mi8;
    if (any_i8 || op == kOpCame) xcd_order(lists[kListAll], desc);
    const int32_t m = static_cast<int32_t>(desc.size());
    size_t total = (m * sizeof(TDesc) + 255) / 256 * 256;
    for (int l = 0; l < kListCount; ++l) {
        out->offs[l] = total;
        out->count[l] = static_cast<int64_t>(lists[l].size());
        total += (lists[l].size() * sizeof(int2) + 255) / 256 * 256;
    }
    total = std::max<size_t>(total, 256);
    out->bytes.assign(total, 0);
    if (m) std::memcpy(out->bytes.data(), desc.data(), m * sizeof(TDesc));
    for (int l = 0; l < kListCount; ++l)
        if (!lists[l].empty())
            std::memcpy(out->bytes.data() + out->offs[l], lists[l].data(), lists[l].size() * sizeof(int2));
    out->n = m;
    out->storage = storage_class(desc);
    return MEO_OK;
}

// Points a Plan's tables into device memory holding a HostPlan's bytes.
void bind_plan(const HostPlan& h, void* dev_bytes, Plan* p) {
    uint8_t* base = static_cast<uint8_t*>(dev_bytes);
    p->n = h.n;
    p->storage = h.storage;
    p->desc = reinterpret_cast<const TDesc*>(base);
    for (int l = 0; l < kListCount; ++l) {
        p->items[l] = reinterpret_cast<const int2*>(base + h.offs[l]);
        p->count[l] = h.count[l];
    }
}

// Builds (or finds) the device-resident launch tables for this list (allocated
// once per distinct list and cached). Returns nullptr with g_err set on a failure.
// `shards` (row-sharded steps; else null): the whole tensors' sizes, part of the key.
Plan* get_plan(int op, int32_t n, const meo_tensor* ts, const StatePtrs* sp, int has_m, int* rc,
               const meo_shard* shards = nullptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        *rc = fail(MEO_EHIP, "hipGetDevice failed");
        return nullptr;
    }
    std::vector<uint8_t> key = plan_key(op, n, ts, sp, has_m, dev, shards);
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto it = g_plans.begin(); it != g_plans.end(); ++it) {
        if ((*it)->key == key) {
            Plan* p = *it;
            g_plans.erase(it);
            g_plans.push_front(p);
            return p;
        }
    }
    HostPlan h;
    *rc = build_host_plan(op, n, ts, sp, has_m, dev, shards, &h);
    if (*rc) return nullptr;
    Plan* p = new Plan;
    p->key = std::move(key);
    p->device = dev;
    if (hipMalloc(&p->mem, h.bytes.size()) != hipSuccess ||
        hipMemcpy(p->mem, h.bytes.data(), h.bytes.size(), hipMemcpyHostToDevice) != hipSuccess) {
        if (p->mem) (void)hipFree(p->mem);
        delete p;
        *rc = fail(MEO_EHIP, "could not allocate or upload the launch table");
        return nullptr;
    }
    bind_plan(h, p->mem, p);
    g_plans.push_front(p);
    while (g_plans.size() > kMaxPlans) {
        free_plan(g_plans.back());
        g_plans.pop_back();
    }
    return p;
}

std::vector<StatePtrs> state_ptrs(int op, int32_t n, const void* states) {
    std::vector<StatePtrs> out(n);
    for (int32_t k = 0; k < n; ++k) {
        StatePtrs& sp = out[k];
        if (op == kOpAdafactor) {
            const auto& s = static_cast<const meo_adafactor_state*>(states)[k];
            sp.m = s.exp_avg; sp.v = s.exp_avg_sq; sp.r = s.exp_avg_sq_row; sp.c = s.exp_avg_sq_col;
            sp.ms = s.exp_avg_scale;
            sp.xsq = s.param_sumsq;
        } else if (op == kOpCame) {
            const auto& s = static_cast<const meo_came_state*>(states)[k];
            sp.m = s.exp_avg; sp.v = s.exp_avg_sq; sp.r = s.exp_avg_sq_row; sp.c = s.exp_avg_sq_col;
            sp.ms = s.exp_avg_scale;
            sp.rr = s.exp_avg_res_row; sp.rc = s.exp_avg_res_col;
        } else {
            const auto& s = static_cast<const meo_lamb_state*>(states)[k];
            sp.m = s.exp_avg; sp.v = s.exp_avg_sq; sp.ms = s.exp_avg_scale;
        }
    }
    return out;
}

// ----------------------------------------------------------------------------- pass timing

enum Pass { kPassStats = 0, kPassFinalize, kPassRms, kPassScalars, kPassAfApply, kPassCameMom,
            kPassCameApply, kPassLambMoments, kPassLambApply, kPassStatsWide, kPassStatsTiled,
            kPassGaProject, kPassGaBack, kPassGaAdamw, kPassGaRefresh, kPassXnorm, kPassSumsqFold, kPassCount };
static_assert(kPassCount == MEO_NUM_PASSES, "pass table");
const char* const kPassNames[kPassCount] = {"stats", "finalize", "rms", "scalars", "adafactor_apply",
                                            "came_mom", "came_apply", "lamb_moments", "lamb_apply",
                                            "stats_wide", "stats_tiled", "galore_project", "galore_back",
                                            "galore_adamw", "galore_refresh", "xnorm", "sumsq_fold"};

struct ProfRec { int pass; hipEvent_t a, b; };
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {
    if (!g_event_pool.empty()) {
        hipEvent_t e = g_event_pool.back();
        g_event_pool.pop_back();
        return e;
    }
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) return nullptr;
    return e;
}

// Records an event after each pass of one step call when profiling is on.
class PassTimer {
  public:
    explicit PassTimer(hipStream_t s) : s_(s) {
        std::lock_guard<std::mutex> lock(g_prof_mu);
        on_ = g_prof_on;
        if (on_) {
            last_ = take_event();
            if (!last_ || hipEventRecord(last_, s_) != hipSuccess) on_ = false;
        }
    }
    void mark(int pass) {
        if (!on_) return;
        std::lock_guard<std::mutex> lock(g_prof_mu);
        hipEvent_t e = take_event();
        if (!e || hipEventRecord(e, s_) != hipSuccess) { on_ = false; return; }
        g_prof.push_back(ProfRec{pass, last_, e});
        last_ = e;
    }
  private:
    hipStream_t s_;
    bool on_ = false;
    hipEvent_t last_ = nullptr;
};

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(MEO_EHIP, std::string(what) + ": " + hipGetErrorString(e));
    return MEO_OK;
}

}  // namespace

// ============================================================================= exports

extern "C" {

const char* meo_last_error(void) { return g_err.c_str(); }

int meo_version(void) { return MEO_VERSION; }

int meo_profile_enable(int on) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_on = on != 0;
    return MEO_OK;
}

const char* meo_pass_name(int id) { return (id >= 0 && id < kPassCount) ? kPassNames[id] : ""; }

int meo_profile_collect(double* total_ms, int64_t* launches) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    int rc = MEO_OK;
    std::vector<hipEvent_t> seen;
    for (const ProfRec& r : g_prof) {
        float ms = 0.0f;
        if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) {
            rc = fail(MEO_EHIP, "could not read pass timing events");
        } else {
            if (total_ms) total_ms[r.pass] += ms;
            if (launches) launches[r.pass] += 1;
        }
        seen.push_back(r.a);
        seen.push_back(r.b);
    }
    std::sort(seen.begin(), seen.end());
    seen.erase(std::unique(seen.begin(), seen.end()), seen.end());
    for (hipEvent_t e : seen) g_event_pool.push_back(e);
    g_prof.clear();
    return rc;
}

void meo_release_plans(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    for (Plan* p : g_plans) free_plan(p);
    g_plans.clear();
    release_galore_plans();
}

// ----------------------------------------------------------------------------- Adafactor

void meo_adafactor_defaults(meo_adafactor_hparams* hp) {
    if (!hp) return;
    std::memset(hp, 0, sizeof *hp);
    hp->lr = 0.0;
    hp->has_lr = 0;
    hp->eps1 = 1e-30;
    hp->eps2 = 1e-3;
    hp->clip_threshold = 1.0;
    hp->decay_rate = -0.8;
    hp->beta1 = 0.0;
    hp->has_beta1 = 0;
    hp->weight_decay = 0.0;
    hp->scale_parameter = 1;
    hp->relative_step = 1;
    hp->warmup_init = 0;
}

size_t meo_adafactor_workspace_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(layout(kOpAdafactor, n, ts, nullptr)) * sizeof(float);
}

int meo_adafactor_scalar_offsets(int32_t n, const meo_tensor* ts, int64_t* offsets) {
    return scalar_offsets(kOpAdafactor, n, ts, offsets);
}

int meo_adafactor_validate(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                           const meo_adafactor_state* st) {
    g_err.clear();
    int rc = check_adafactor_hp(hp);
    if (rc) return rc;
    rc = check_tensors(kOpAdafactor, step, n, ts, st);
    if (rc) return rc;
    if (hp->has_beta1)
        for (int32_t k = 0; k < n; ++k) {
            rc = check_moment(kOpAdafactor, k, ts[k], st[k].exp_avg, st[k].exp_avg_scale, " but beta1 is set");
            if (rc) return rc;
        }
    return MEO_OK;
}

}  // extern "C"

namespace {

// Every tensor with elements has a 4-byte aligned param_sumsq (the carry calls).
int check_param_sumsq(int32_t n, const meo_tensor* ts, const meo_adafactor_state* st) {
    for (int32_t k = 0; k < n; ++k) {
        int64_t numel = 0;
        overflow_numel(ts[k], &numel);
        if (numel == 0) continue;
        if (!st[k].param_sumsq) return fail(MEO_ENULL, "tensor " + std::to_string(k) + ": param_sumsq is NULL");
        if (reinterpret_cast<uintptr_t>(st[k].param_sumsq) % 4)
            return fail(MEO_EALIGN, "tensor " + std::to_string(k) + ": param_sumsq misaligned");
    }
    return MEO_OK;
}

int adafactor_passes(const meo_adafactor_hparams* hp, int64_t step, int carry, const Plan& plan, float* w,
                     hipStream_t s);

// carry: -1 plain step; 0 or 1 a step that leaves the updated parameter's sum of
// squares in each tensor's param_sumsq (1: and takes RMS(X) from it).
int adafactor_step(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                   const meo_adafactor_state* st, int carry, void* ws, size_t ws_bytes, void* stream) {
    int rc = meo_adafactor_validate(hp, step, n, ts, st);
    if (rc) return rc;
    // RMS(X) is needed only to scale the step (scale_parameter); without it the
    // carried sum is neither read nor written.
    if (!hp->scale_parameter) carry = -1;
    if (carry >= 0) {
        rc = check_param_sumsq(n, ts, st);
        if (rc) return rc;
    }
    if (n == 0) return MEO_OK;
    rc = check_workspace(kOpAdafactor, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpAdafactor, n, st);
    Plan* p = get_plan(kOpAdafactor, n, ts, sp.data(), hp->has_beta1, &rc);
    if (!p) return rc;
    if (p->n == 0) return MEO_OK;
    return adafactor_passes(hp, step, carry, *p, static_cast<float*>(ws), static_cast<hipStream_t>(stream));
}

// The passes of one Adafactor step over a list whose launch tables are `p` and
// whose workspace starts at `w`, enqueued on `s`. carry as for adafactor_step.
int adafactor_passes(const meo_adafactor_hparams* hp, int64_t step, int carry, const Plan& plan, float* w,
                     hipStream_t s) {
    const Plan* p = &plan;
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };

    const double tt = static_cast<double>(step);
    double rho;
    if (hp->relative_step) rho = std::fmin(hp->warmup_init ? 1e-6 * tt : 1e-2, 1.0 / std::sqrt(tt));
    else rho = hp->lr;
    const double b2 = 1.0 - std::pow(tt, hp->decay_rate);
    // The first pass reads X for RMS(X) unless the carried sums stand for it.
    const int32_t need_x = hp->scale_parameter && carry != 1 ? 1 : 0;
    const StatsArgs sa{static_cast<float>(hp->eps1), static_cast<float>(b2), static_cast<float>(1.0 - b2), need_x,
                       b2, 1.0 - b2};

    PassTimer pt(s);
    if (need_x && p->count[kListXnorm]) {
        launch_xnorm(tab(kListXnorm), p->count[kListXnorm], sa, s);
        pt.mark(kPassXnorm);
    }
    if (p->count[kListRc0]) {
        launch_rowstats(0, tab(kListRc0), p->count[kListRc0], sa, s);
        pt.mark(kPassStats);
    }
    if (p->count[kListRc1]) {
        launch_rowstats(1, tab(kListRc1), p->count[kListRc1], sa, s);
        pt.mark(kPassStatsWide);
    }
    if (p->count[kListTiled]) {
        launch_stats(tab(kListTiled), p->count[kListTiled], sa, s);
        pt.mark(kPassStatsTiled);
    }
    launch_finalize(tab(kListFin1), p->count[kListFin1], FinArgs{b2, 0, 0}, s);
    pt.mark(kPassFinalize);
    if (p->count[kListTiled]) {
        launch_rms(tab(kListTiled), p->count[kListTiled], need_x, s);
        pt.mark(kPassRms);
    }
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalAdafactor, hp->scale_parameter, nullptr, carry == 1 ? 1 : 0,
                                              rho, hp->eps2, hp->clip_threshold, hp->weight_decay, 0.0}, s);
    pt.mark(kPassScalars);
    launch_af_apply(tab(kListAll), p->count[kListAll],
                    AfApplyArgs{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1), hp->has_beta1},
                    p->storage, carry >= 0, s);
    pt.mark(kPassAfApply);
    if (carry >= 0) {
        launch_sumsq_fold(p->desc, w, p->n, s);
        pt.mark(kPassSumsqFold);
    }
    return launch_status("adafactor step launch");
}

}  // namespace

extern "C" {

int meo_adafactor_step(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                       const meo_adafactor_state* st, void* ws, size_t ws_bytes, void* stream) {
    return adafactor_step(hp, step, n, ts, st, -1, ws, ws_bytes, stream);
}

int meo_adafactor_step_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                             const meo_adafactor_state* st, int32_t param_sumsq_valid, void* ws, size_t ws_bytes,
                             void* stream) {
    return adafactor_step(hp, step, n, ts, st, param_sumsq_valid ? 1 : 0, ws, ws_bytes, stream);
}

// ----------------------------------------------------------------------------- no-allocation step

// Scratch of meo_adafactor_step_noalloc: one call's launch tables followed by its
// workspace. A file-scope device array, so the library never allocates it: each
// GPU that loads this code holds its own copy until the process ends. Host code
// must not pass the array's name to a kernel (it stands for a host-side shadow);
// the device address of each GPU's copy comes from hipGetSymbolAddress.
__device__ __align__(256) unsigned char scratch[MEO_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_na_mu;
std::vector<void*> g_scratch_ptr;  // per device, filled on the first call on it
// Host launch tables of recent lists (most recent first), for the no-allocation step.
std::list<std::pair<std::vector<uint8_t>, HostPlan>> g_na_plans;
constexpr size_t kMaxNaPlans = 16;

// The device address of this device's scratch (looked up once per device, with the
// device current). Call with g_na_mu held.
void* scratch_of(int dev, int* rc) {
    if (static_cast<size_t>(dev) >= g_scratch_ptr.size()) g_scratch_ptr.resize(dev + 1, nullptr);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !ptr) {
            *rc = fail(MEO_EHIP, std::string("hipGetSymbolAddress of the scratch array failed: ") +
                                     hipGetErrorString(e));
            return nullptr;
        }
        g_scratch_ptr[dev] = ptr;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

int meo_adafactor_step_noalloc(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                               const meo_adafactor_state* st, void* stream) {
    int rc = meo_adafactor_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    const size_t ws_bytes = static_cast<size_t>(layout(kOpAdafactor, n, ts, nullptr)) * sizeof(float);
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return fail(MEO_EHIP, "hipGetDevice failed");
    const std::vector<StatePtrs> sp = state_ptrs(kOpAdafactor, n, st);
    std::vector<uint8_t> key = plan_key(kOpAdafactor, n, ts, sp.data(), hp->has_beta1, dev, nullptr);
    const hipStream_t s = static_cast<hipStream_t>(stream);
    std::lock_guard<std::mutex> lock(g_na_mu);
    auto it = g_na_plans.begin();
    for (; it != g_na_plans.end(); ++it)
        if (it->first == key) break;
    if (it == g_na_plans.end()) {
        HostPlan h;
        rc = build_host_plan(kOpAdafactor, n, ts, sp.data(), hp->has_beta1, dev, nullptr, &h);
        if (rc) return rc;
        g_na_plans.emplace_front(std::move(key), std::move(h));
        if (g_na_plans.size() > kMaxNaPlans) g_na_plans.pop_back();
    } else if (it != g_na_plans.begin()) {
        g_na_plans.splice(g_na_plans.begin(), g_na_plans, it);
    }
    const HostPlan& h = g_na_plans.front().second;
    const size_t tbytes = (h.bytes.size() + 255) / 256 * 256;
    if (tbytes + ws_bytes > MEO_NOALLOC_SCRATCH_BYTES)
        return fail(MEO_EWORKSPACE, "this list needs " + std::to_string(tbytes + ws_bytes) +
                                        " bytes of scratch (launch tables and workspace); "
                                        "meo_adafactor_step_noalloc holds at most " +
                                        std::to_string(static_cast<size_t>(MEO_NOALLOC_SCRATCH_BYTES)) +
                                        " (meo_adafactor_step takes a workspace of any size)");
    if (h.n == 0) return MEO_OK;
    uint8_t* base = static_cast<uint8_t*>(scratch_of(dev, &rc));
    if (!base) return rc;
    // The tables go in on the stream, before the passes that read them. The host
    // bytes stay in the cache; a pageable source is consumed before the call returns.
    const hipError_t e = hipMemcpyAsync(base, h.bytes.data(), h.bytes.size(), hipMemcpyHostToDevice, s);
    if (e != hipSuccess) return fail(MEO_EHIP, std::string("launch table upload: ") + hipGetErrorString(e));
    Plan view;
    bind_plan(h, base, &view);
    return adafactor_passes(hp, step, -1, view, reinterpret_cast<float*>(base + tbytes), s);
}

}  // extern "C"

// ----------------------------------------------------------------------------- CAME

void meo_came_defaults(meo_came_hparams* hp) {
    if (!hp) return;
    std::memset(hp, 0, sizeof *hp);
    hp->lr = 0.0;
    hp->has_lr = 0;
    hp->eps1 = 1e-30;
    hp->eps2 = 1e-16;
    hp->clip_threshold = 1.0;
    hp->beta1 = 0.9;
    hp->beta2 = 0.999;
    hp->beta3 = 0.9999;
    hp->weight_decay = 0.0;
}

size_t meo_came_workspace_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(layout(kOpCame, n, ts, nullptr)) * sizeof(float);
}

int meo_came_scalar_offsets(int32_t n, const meo_tensor* ts, int64_t* offsets) {
    return scalar_offsets(kOpCame, n, ts, offsets);
}

int meo_came_validate(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                      const meo_came_state* st) {
    g_err.clear();
    int rc = check_came_hp(hp);
    if (rc) return rc;
    rc = check_tensors(kOpCame, step, n, ts, st);
    if (rc) return rc;
    for (int32_t k = 0; k < n; ++k) {
        rc = check_moment(kOpCame, k, ts[k], st[k].exp_avg, st[k].exp_avg_scale, "");
        if (rc) return rc;
    }
    return MEO_OK;
}

int meo_came_step(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                  const meo_came_state* st, void* ws, size_t ws_bytes, void* stream) {
    int rc = meo_came_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_workspace(kOpCame, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpCame, n, st);
    Plan* p = get_plan(kOpCame, n, ts, sp.data(), 1, &rc);
    if (!p) return rc;
    if (p->n == 0) return MEO_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    const StatsArgs sa{static_cast<float>(hp->eps1), static_cast<float>(hp->beta2),
                       static_cast<float>(1.0 - hp->beta2), 0, hp->beta2, 1.0 - hp->beta2};

    PassTimer pt(s);
    if (p->count[kListRc0]) {
        launch_rowstats(0, tab(kListRc0), p->count[kListRc0], sa, s);
        pt.mark(kPassStats);
    }
    if (p->count[kListRc1]) {
        launch_rowstats(1, tab(kListRc1), p->count[kListRc1], sa, s);
        pt.mark(kPassStatsWide);
    }
    if (p->count[kListTiled]) {
        launch_stats(tab(kListTiled), p->count[kListTiled], sa, s);
        pt.mark(kPassStatsTiled);
    }
    launch_finalize(tab(kListFin1), p->count[kListFin1], FinArgs{hp->beta2, 0, 0}, s);
    pt.mark(kPassFinalize);
    if (p->count[kListTiled]) {
        launch_rms(tab(kListTiled), p->count[kListTiled], 0, s);
        pt.mark(kPassRms);
    }
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalCame1, 0, nullptr, 0, 0.0, 0.0, hp->clip_threshold, hp->weight_decay,
                                              hp->lr}, s);
    pt.mark(kPassScalars);
    launch_came_mom(tab(kListAll), p->count[kListAll],
                    CameArgs{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1),
                             static_cast<float>(hp->eps2), static_cast<float>(hp->lr)},
                    p->storage, s);
    pt.mark(kPassCameMom);
    launch_finalize(tab(kListFin2), p->count[kListFin2], FinArgs{hp->beta3, 1, 1}, s);
    pt.mark(kPassFinalize);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalCame2, 0, nullptr, 0, 0.0, 0.0, hp->clip_threshold, hp->weight_decay,
                                              hp->lr}, s);
    pt.mark(kPassScalars);
    launch_came_apply(tab(kListCameApply), p->count[kListCameApply], p->storage, s);
    pt.mark(kPassCameApply);
    return launch_status("came step launch");
}

// ----------------------------------------------------------------------------- LAMB

void meo_lamb_defaults(meo_lamb_hparams* hp) {
    if (!hp) return;
    std::memset(hp, 0, sizeof *hp);
    hp->lr = 1e-3;
    hp->beta1 = 0.9;
    hp->beta2 = 0.999;
    hp->eps = 1e-6;
    hp->weight_decay = 0.0;
    hp->bias_correction = 1;
}

size_t meo_lamb_workspace_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(layout(kOpLamb, n, ts, nullptr)) * sizeof(float);
}

int meo_lamb_scalar_offsets(int32_t n, const meo_tensor* ts, int64_t* offsets) {
    return scalar_offsets(kOpLamb, n, ts, offsets);
}

int meo_lamb_validate(const meo_lamb_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                      const meo_lamb_state* st) {
    g_err.clear();
    int rc = check_lamb_hp(hp);
    if (rc) return rc;
    rc = check_tensors(kOpLamb, step, n, ts, st);
    if (rc) return rc;
    for (int32_t k = 0; k < n; ++k) {
        rc = check_moment(kOpLamb, k, ts[k], st[k].exp_avg, st[k].exp_avg_scale, "");
        if (rc) return rc;
    }
    return MEO_OK;
}

int meo_lamb_step(const meo_lamb_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                  const meo_lamb_state* st, void* ws, size_t ws_bytes, void* stream) {
    int rc = meo_lamb_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_workspace(kOpLamb, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpLamb, n, st);
    Plan* p = get_plan(kOpLamb, n, ts, sp.data(), 1, &rc);
    if (!p) return rc;
    if (p->n == 0) return MEO_OK;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* w = static_cast<float*>(ws);
    const Table t{p->desc, p->items[kListAll], w};
    const int64_t tiles = p->count[kListAll];

    const double tt = static_cast<double>(step);
    const double bc1 = hp->bias_correction ? 1.0 - std::pow(hp->beta1, tt) : 1.0;
    const double bc2 = hp->bias_correction ? 1.0 - std::pow(hp->beta2, tt) : 1.0;
    const LambArgs la{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1),
                      static_cast<float>(hp->beta2), static_cast<float>(1.0 - hp->beta2),
                      static_cast<float>(1.0 / bc1), static_cast<float>(1.0 / bc2),
                      static_cast<float>(hp->eps), static_cast<float>(hp->weight_decay)};
    PassTimer pt(s);
    launch_lamb_moments(t, tiles, la, p->storage, s);
    pt.mark(kPassLambMoments);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalLamb, 0, nullptr, 0, 0.0, 0.0, 1.0, hp->weight_decay, hp->lr}, s);
    pt.mark(kPassScalars);
    launch_lamb_apply(t, tiles, la, p->storage, s);
    pt.mark(kPassLambApply);
    return launch_status("lamb step launch");
}


// ----------------------------------------------------------------------------- row-sharded steps

namespace {

// The shard sizes and the partial-sum buffer: factored shards need row-complete
// rows (the single exchange rests on whole rows), the whole tensor is at least the
// shard, and the buffer is device memory of the record's size.
// A record buffer: device memory of `floats` floats, 4-byte aligned.
int check_record(const void* p, int64_t floats, const char* name) {
    if (floats == 0) return MEO_OK;
    if (!p) return fail(MEO_ENULL, std::string(name) + " is NULL");
    if (reinterpret_cast<uintptr_t>(p) % 4) return fail(MEO_EALIGN, std::string(name) + " not 4-byte aligned");
    if (floats > kMaxDim) return fail(MEO_ESHAPE, std::string("the record ") + name + " exceeds 2^31 - 1 floats");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MEO_EHIP, "hipGetDevice failed");
    }
    return check_device_range(p, static_cast<size_t>(floats) * 4, dev, name, MEO_EMEMORY);
}

int check_shards(int op, int32_t n, const meo_tensor* ts, const meo_shard* sh, const void* partials,
                 bool with_partials = true) {
    if (n == 0) return MEO_OK;
    if (!sh) return fail(MEO_ENULL, "shards is NULL");
    if (with_partials && !partials) return fail(MEO_ENULL, "partials is NULL");
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        int64_t numel = 0;
        overflow_numel(t, &numel);
        if (numel == 0) continue;
        const std::string who = "tensor " + std::to_string(k) + ": ";
        if (is_factored(op, t)) {
            if (sh[k].rows_total < t.rows || sh[k].rows_total > kMaxDim)
                return fail(MEO_ESHAPE, who + "rows_total must be >= the shard's rows and < 2^31");
            if (t.cols % kVec != 0 || t.cols > kRcMaxCols1 || !aligned16(t.param) || !aligned16(t.grad))
                return fail(MEO_ESHAPE, who + "a row-sharded factored tensor needs cols % 8 == 0, cols <= " +
                                            std::to_string(kRcMaxCols1) + " and 16-byte aligned param and grad");
        } else if (sh[k].rows_total < numel) {
            return fail(MEO_ESHAPE, who + "rows_total (elements of the whole tensor) must be >= the shard's");
        }
    }
    if (!with_partials) return MEO_OK;
    return check_record(partials, partials_layout(op, n, ts, nullptr), "partials");
}

struct AfShard {
    Plan* p = nullptr;
    double rho = 0.0, b2 = 0.0;
};

int af_shard_prepare(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                     const meo_shard* sh, const meo_adafactor_state* st, const void* partials, void* ws,
                     size_t ws_bytes, AfShard* out, bool carry = false) {
    int rc = meo_adafactor_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (carry && hp->scale_parameter) {
        rc = check_param_sumsq(n, ts, st);
        if (rc) return rc;
    }
    if (n == 0) return MEO_OK;
    rc = check_shards(kOpAdafactor, n, ts, sh, partials);
    if (rc) return rc;
    rc = check_workspace(kOpAdafactor, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpAdafactor, n, st);
    out->p = get_plan(kOpAdafactor, n, ts, sp.data(), hp->has_beta1, &rc, sh);
    if (!out->p) return rc;
    const double tt = static_cast<double>(step);
    out->rho = hp->relative_step ? std::fmin(hp->warmup_init ? 1e-6 * tt : 1e-2, 1.0 / std::sqrt(tt)) : hp->lr;
    out->b2 = 1.0 - std::pow(tt, hp->decay_rate);
    return MEO_OK;
}

LambArgs lamb_args(const meo_lamb_hparams* hp, int64_t step) {
    const double tt = static_cast<double>(step);
    const double bc1 = hp->bias_correction ? 1.0 - std::pow(hp->beta1, tt) : 1.0;
    const double bc2 = hp->bias_correction ? 1.0 - std::pow(hp->beta2, tt) : 1.0;
    return LambArgs{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1),
                    static_cast<float>(hp->beta2), static_cast<float>(1.0 - hp->beta2),
                    static_cast<float>(1.0 / bc1), static_cast<float>(1.0 / bc2),
                    static_cast<float>(hp->eps), static_cast<float>(hp->weight_decay)};
}

int lamb_shard_prepare(const meo_lamb_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                       const meo_shard* sh, const meo_lamb_state* st, const void* partials, void* ws,
                       size_t ws_bytes, Plan** out) {
    int rc = meo_lamb_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_shards(kOpLamb, n, ts, sh, partials);
    if (rc) return rc;
    rc = check_workspace(kOpLamb, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpLamb, n, st);
    *out = get_plan(kOpLamb, n, ts, sp.data(), 1, &rc, sh);
    return *out ? MEO_OK : rc;
}

}  // namespace

size_t meo_adafactor_partials_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(partials_layout(kOpAdafactor, n, ts, nullptr));
}

size_t meo_lamb_partials_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(partials_layout(kOpLamb, n, ts, nullptr));
}

// carry: -1 plain; 0 or 1 as for the whole-tensor carry call (1: the record's sum
// of X^2 is the shard's carried value and X is not read).
static int af_shard_stats(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                   const meo_shard* sh, const meo_adafactor_state* st, float* partials, int carry, void* ws,
                   size_t ws_bytes, void* stream) {
    AfShard a;
    int rc = af_shard_prepare(hp, step, n, ts, sh, st, partials, ws, ws_bytes, &a, carry >= 0);
    if (rc || n == 0) return rc;
    Plan* p = a.p;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    launch_zero_records(p->items[kListEmpty], p->count[kListEmpty], partials, s);
    if (p->n == 0) return launch_status("adafactor shard statistics launch");
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    const int32_t carried = hp->scale_parameter && carry == 1 ? 1 : 0;
    const int32_t need_x = hp->scale_parameter && !carried ? 1 : 0;
    const StatsArgs sa{static_cast<float>(hp->eps1), static_cast<float>(a.b2), static_cast<float>(1.0 - a.b2), need_x,
                       a.b2, 1.0 - a.b2};
    PassTimer pt(s);
    if (need_x && p->count[kListXnorm]) {
        launch_xnorm(tab(kListXnorm), p->count[kListXnorm], sa, s);
        pt.mark(kPassXnorm);
    }
    if (p->count[kListRc0]) {
        launch_rowstats(0, tab(kListRc0), p->count[kListRc0], sa, s);
        pt.mark(kPassStats);
    }
    if (p->count[kListRc1]) {
        launch_rowstats(1, tab(kListRc1), p->count[kListRc1], sa, s);
        pt.mark(kPassStatsWide);
    }
    launch_shard_partials(tab(kListShard), p->count[kListShard], partials, need_x, carried, s);
    pt.mark(kPassFinalize);
    return launch_status("adafactor shard statistics launch");
}

int meo_adafactor_shard_stats(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                              const meo_shard* sh, const meo_adafactor_state* st, float* partials, void* ws,
                              size_t ws_bytes, void* stream) {
    return af_shard_stats(hp, step, n, ts, sh, st, partials, -1, ws, ws_bytes, stream);
}

int meo_adafactor_shard_stats_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                                    const meo_shard* sh, const meo_adafactor_state* st, int32_t param_sumsq_valid,
                                    float* partials, void* ws, size_t ws_bytes, void* stream) {
    return af_shard_stats(hp, step, n, ts, sh, st, partials, param_sumsq_valid ? 1 : 0, ws, ws_bytes, stream);
}

// carry: also leave the shard's sum of squares of its updated rows in param_sumsq.
static int af_shard_apply(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                   const meo_shard* sh, const meo_adafactor_state* st, const float* partials, bool carry, void* ws,
                   size_t ws_bytes, void* stream) {
    AfShard a;
    int rc = af_shard_prepare(hp, step, n, ts, sh, st, partials, ws, ws_bytes, &a, carry);
    carry = carry && hp->scale_parameter;
    if (rc || n == 0 || a.p->n == 0) return rc;
    Plan* p = a.p;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    PassTimer pt(s);
    launch_shard_fold(tab(kListFold), p->count[kListFold], partials, a.b2, s);
    pt.mark(kPassFinalize);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalAdafactor, hp->scale_parameter, partials, 0, a.rho, hp->eps2,
                                              hp->clip_threshold, hp->weight_decay, 0.0}, s);
    pt.mark(kPassScalars);
    launch_af_apply(tab(kListAll), p->count[kListAll],
                    AfApplyArgs{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1), hp->has_beta1},
                    p->storage, carry, s);
    pt.mark(kPassAfApply);
    if (carry) {
        launch_sumsq_fold(p->desc, w, p->n, s);
        pt.mark(kPassSumsqFold);
    }
    return launch_status("adafactor shard apply launch");
}

int meo_adafactor_shard_apply(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                              const meo_shard* sh, const meo_adafactor_state* st, const float* partials, void* ws,
                              size_t ws_bytes, void* stream) {
    return af_shard_apply(hp, step, n, ts, sh, st, partials, false, ws, ws_bytes, stream);
}

int meo_adafactor_shard_apply_carry(const meo_adafactor_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                                    const meo_shard* sh, const meo_adafactor_state* st, const float* partials,
                                    void* ws, size_t ws_bytes, void* stream) {
    return af_shard_apply(hp, step, n, ts, sh, st, partials, true, ws, ws_bytes, stream);
}

int meo_lamb_shard_stats(const meo_lamb_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                         const meo_shard* sh, const meo_lamb_state* st, float* partials, void* ws, size_t ws_bytes,
                         void* stream) {
    Plan* p = nullptr;
    int rc = lamb_shard_prepare(hp, step, n, ts, sh, st, partials, ws, ws_bytes, &p);
    if (rc || n == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    launch_zero_records(p->items[kListEmpty], p->count[kListEmpty], partials, s);
    if (p->n == 0) return launch_status("lamb shard statistics launch");
    float* w = static_cast<float*>(ws);
    PassTimer pt(s);
    launch_lamb_moments(Table{p->desc, p->items[kListAll], w}, p->count[kListAll], lamb_args(hp, step), p->storage, s);
    pt.mark(kPassLambMoments);
    launch_shard_partials(Table{p->desc, p->items[kListShard], w}, p->count[kListShard], partials, 0, 0, s);
    pt.mark(kPassFinalize);
    return launch_status("lamb shard statistics launch");
}

int meo_lamb_shard_apply(const meo_lamb_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                         const meo_shard* sh, const meo_lamb_state* st, const float* partials, void* ws,
                         size_t ws_bytes, void* stream) {
    Plan* p = nullptr;
    int rc = lamb_shard_prepare(hp, step, n, ts, sh, st, partials, ws, ws_bytes, &p);
    if (rc || n == 0 || p->n == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* w = static_cast<float*>(ws);
    PassTimer pt(s);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalLamb, 0, partials, 0, 0.0, 0.0, 1.0, hp->weight_decay, hp->lr}, s);
    pt.mark(kPassScalars);
    launch_lamb_apply(Table{p->desc, p->items[kListAll], w}, p->count[kListAll], lamb_args(hp, step), p->storage, s);
    pt.mark(kPassLambApply);
    return launch_status("lamb shard apply launch");
}

// ----------------------------------------------------------------------------- CAME, row-sharded

namespace {

int came_shard_prepare(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                       const meo_shard* sh, const meo_came_state* st, const void* partials, bool with_partials,
                       const void* conf, bool with_conf, void* ws, size_t ws_bytes, Plan** out) {
    int rc = meo_came_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_shards(kOpCame, n, ts, sh, partials, with_partials);
    if (rc) return rc;
    if (with_conf) {
        rc = check_record(conf, confidence_layout(n, ts, nullptr), "confidence");
        if (rc) return rc;
    }
    rc = check_workspace(kOpCame, n, ts, ws, ws_bytes);
    if (rc) return rc;
    const std::vector<StatePtrs> sp = state_ptrs(kOpCame, n, st);
    *out = get_plan(kOpCame, n, ts, sp.data(), 1, &rc, sh);
    return *out ? MEO_OK : rc;
}

}  // namespace

size_t meo_came_partials_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(partials_layout(kOpCame, n, ts, nullptr));
}

size_t meo_came_confidence_size(int32_t n, const meo_tensor* ts) {
    if (n <= 0 || !ts) return 0;
    return static_cast<size_t>(confidence_layout(n, ts, nullptr));
}

int meo_came_shard_stats(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                         const meo_shard* sh, const meo_came_state* st, float* partials, void* ws, size_t ws_bytes,
                         void* stream) {
    Plan* p = nullptr;
    int rc = came_shard_prepare(hp, step, n, ts, sh, st, partials, true, nullptr, false, ws, ws_bytes, &p);
    if (rc || n == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    launch_zero_records(p->items[kListEmpty], p->count[kListEmpty], partials, s);
    if (p->n == 0) return launch_status("came shard statistics launch");
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    const StatsArgs sa{static_cast<float>(hp->eps1), static_cast<float>(hp->beta2),
                       static_cast<float>(1.0 - hp->beta2), 0, hp->beta2, 1.0 - hp->beta2};
    PassTimer pt(s);
    if (p->count[kListRc0]) {
        launch_rowstats(0, tab(kListRc0), p->count[kListRc0], sa, s);
        pt.mark(kPassStats);
    }
    if (p->count[kListRc1]) {
        launch_rowstats(1, tab(kListRc1), p->count[kListRc1], sa, s);
        pt.mark(kPassStatsWide);
    }
    launch_shard_partials(tab(kListShard), p->count[kListShard], partials, 0, 0, s);
    pt.mark(kPassFinalize);
    return launch_status("came shard statistics launch");
}

int meo_came_shard_moment(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                          const meo_shard* sh, const meo_came_state* st, const float* partials, float* conf,
                          void* ws, size_t ws_bytes, void* stream) {
    Plan* p = nullptr;
    int rc = came_shard_prepare(hp, step, n, ts, sh, st, partials, true, conf, true, ws, ws_bytes, &p);
    if (rc || n == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    launch_zero_records(p->items[kListEmpty2], p->count[kListEmpty2], conf, s);
    if (p->n == 0) return launch_status("came shard moment launch");
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    PassTimer pt(s);
    launch_shard_fold(tab(kListFold), p->count[kListFold], partials, hp->beta2, s);
    pt.mark(kPassFinalize);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalCame1, 0, partials, 0, 0.0, 0.0, hp->clip_threshold,
                                              hp->weight_decay, hp->lr}, s);
    pt.mark(kPassScalars);
    launch_came_mom(tab(kListAll), p->count[kListAll],
                    CameArgs{static_cast<float>(hp->beta1), static_cast<float>(1.0 - hp->beta1),
                             static_cast<float>(hp->eps2), static_cast<float>(hp->lr)},
                    p->storage, s);
    pt.mark(kPassCameMom);
    // the confidence row statistic is local (whole rows); its column sums are not
    launch_finalize(tab(kListConfRows), p->count[kListConfRows], FinArgs{hp->beta3, 1, 1}, s);
    launch_conf_partials(tab(kListConf), p->count[kListConf], conf, s);
    pt.mark(kPassFinalize);
    return launch_status("came shard moment launch");
}

int meo_came_shard_apply(const meo_came_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                         const meo_shard* sh, const meo_came_state* st, const float* conf, void* ws,
                         size_t ws_bytes, void* stream) {
    Plan* p = nullptr;
    int rc = came_shard_prepare(hp, step, n, ts, sh, st, nullptr, false, conf, true, ws, ws_bytes, &p);
    if (rc || n == 0 || p->n == 0) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    float* w = static_cast<float*>(ws);
    auto tab = [&](int l) { return Table{p->desc, p->items[l], w}; };
    PassTimer pt(s);
    launch_conf_fold(tab(kListConf), p->count[kListConf], conf, hp->beta3, s);
    pt.mark(kPassFinalize);
    launch_scalars(p->desc, w, p->n, ScalArgs{kScalCame2, 0, conf, 0, 0.0, 0.0, hp->clip_threshold, hp->weight_decay,
                                              hp->lr}, s);
    pt.mark(kPassScalars);
    launch_came_apply(tab(kListCameApply), p->count[kListCameApply], p->storage, s);
    pt.mark(kPassCameApply);
    return launch_status("came shard apply launch");
}

// ----------------------------------------------------------------------------- GaLore

namespace {

enum GaList { kGaProjR = 0, kGaProjL, kGaBackR, kGaBackL, kGaFlat,
              // projector refresh
              kRfInit, kRfG0N, kRfG0T, kRfG1N, kRfG1T, kRfGram, kRfOne, kRfCols, kRfStore, kGaListCount };

struct GaPlan {
    std::vector<uint8_t> key;
    int device = 0;
    void* mem = nullptr;  // [GDesc right..., left...][TDesc flat...][RDesc...][item tables]
    const GDesc* gdesc = nullptr;
    const TDesc* fdesc = nullptr;
    const RDesc* rdesc = nullptr;
    const int2* items[kGaListCount] = {};
    int64_t count[kGaListCount] = {};
    int back_mode[2] = {kBackReg, kBackReg};  // back-projection kernel (BackMode), right and left
    bool proj_direct[2] = {false, false};  // projection staged by global_load_lds (right, left)
    int nright = 0;  // right-side descriptors, first in gdesc
};
std::list<GaPlan*> g_ga_plans;  // most recently used first, under g_mu

void release_galore_plans() {  // caller holds g_mu
    for (GaPlan* p : g_ga_plans) {
        int cur = 0;
        (void)hipGetDevice(&cur);
        if (cur != p->device) (void)hipSetDevice(p->device);
        (void)hipFree(p->mem);
        if (cur != p->device) (void)hipSetDevice(cur);
        delete p;
    }
    g_ga_plans.clear();
}

bool ga_projected(const meo_tensor& t) { return t.ndim == 2 && t.rows > 0 && t.cols > 0; }

int32_t ga_rank(const meo_galore_hparams* hp, const meo_tensor& t) {
    if (!ga_projected(t)) return 0;
    return static_cast<int32_t>(std::min<int64_t>(hp->rank, std::min(t.rows, t.cols)));
}

// The projected side: left (R = P^T G, P from the left singular vectors) or right.
// std takes the shorter side, reverse_std the longer one.
bool ga_left(const meo_galore_hparams* hp, const meo_tensor& t) {
    return (t.rows < t.cols) == (hp->proj_type == MEO_GALORE_STD);
}
int64_t ga_rows(const meo_galore_hparams* hp, const meo_tensor& t) { return ga_left(hp, t) ? t.cols : t.rows; }   // D
int64_t ga_basis(const meo_galore_hparams* hp, const meo_tensor& t) { return ga_left(hp, t) ? t.rows : t.cols; }  // d

int64_t align256(int64_t bytes) { return (bytes + 255) / 256 * 256; }

// Workspace, per projected tensor, every array at a 256-byte boundary (offsets in
// bytes): the step's two bf16 planes of N, [D][r] each; then, for the projector
// refresh, two fp32 [r][d] iterates, one fp32 [r][D] product, and four fp64
// [r][r] matrices.
int64_t ga_layout(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts, std::vector<int64_t>* offs,
                  std::vector<int64_t>* roffs = nullptr) {
    int64_t off = 0;
    if (offs) offs->assign(n, -1);
    if (roffs) roffs->assign(n, -1);
    for (int32_t k = 0; k < n; ++k) {
        const int32_t r = ga_rank(hp, ts[k]);
        if (!r) continue;
        if (offs) (*offs)[k] = off;
        off += 2 * align256(ga_rows(hp, ts[k]) * r * 2);
    }
    for (int32_t k = 0; k < n; ++k) {
        const int32_t r = ga_rank(hp, ts[k]);
        if (!r) continue;
        if (roffs) (*roffs)[k] = off;
        const int64_t d = ga_basis(hp, ts[k]), D = ga_rows(hp, ts[k]);
        // the product buffer [r][D] later holds the basis [r][d] too
        off += 2 * align256(static_cast<int64_t>(r) * d * 4) + align256(static_cast<int64_t>(r) * std::max(D, d) * 4) +
               4 * align256(static_cast<int64_t>(r) * r * 8);
    }
    return off;
}

int check_galore_hp(const meo_galore_hparams* hp) {
    if (!hp) return fail(MEO_ENULL, "hparams is NULL");
    if (!finite(hp->lr) || !finite(hp->beta1) || !finite(hp->beta2) || !finite(hp->eps) ||
        !finite(hp->weight_decay) || !finite(hp->scale))
        return fail(MEO_EINVAL, "non-finite hyperparameter");
    if (hp->lr < 0.0) return fail(MEO_EINVAL, "Invalid learning rate: " + std::to_string(hp->lr));
    if (hp->beta1 < 0.0 || hp->beta1 >= 1.0 || hp->beta2 < 0.0 || hp->beta2 >= 1.0)
        return fail(MEO_EINVAL, "betas must lie in [0, 1)");
    if (hp->eps < 0.0) return fail(MEO_EINVAL, "Invalid epsilon value: " + std::to_string(hp->eps));
    if (hp->rank < 1) return fail(MEO_EINVAL, "rank must be >= 1");
    if (hp->update_proj_gap < 1) return fail(MEO_EINVAL, "update_proj_gap must be >= 1");
    if (hp->proj_type != MEO_GALORE_STD && hp->proj_type != MEO_GALORE_REVERSE_STD)
        return fail(MEO_EINVAL, "proj_type must be MEO_GALORE_STD or MEO_GALORE_REVERSE_STD");
    return MEO_OK;
}

int check_galore_tensors(const meo_galore_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                         const meo_galore_state* st) {
    if (step < 1) return fail(MEO_EINVAL, "step must be >= 1 (1-based index of the step being taken)");
    if (n < 0) return fail(MEO_EINVAL, "negative tensor count");
    if (n == 0) return MEO_OK;
    if (!ts) return fail(MEO_ENULL, "tensors is NULL");
    if (!st) return fail(MEO_ENULL, "states is NULL");
    int64_t blocks[kGaListCount] = {};
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        const std::string who = "tensor " + std::to_string(k) + ": ";
        if (t.batch < 0 || t.rows < 0 || t.cols < 0 || t.ndim < 0)
            return fail(MEO_ESHAPE, who + "negative batch, rows, cols or ndim");
        int64_t numel;
        if (overflow_numel(t, &numel)) return fail(MEO_ESHAPE, who + "too many elements");
        if (t.ndim <= 1 && numel > 0 && (t.batch != 1 || t.rows != 1))
            return fail(MEO_ESHAPE, who + "a tensor with ndim <= 1 must have batch == rows == 1");
        if (t.ndim == 2 && numel > 0 && t.batch != 1) return fail(MEO_ESHAPE, who + "a 2-D tensor has batch 1");
        if (t.param_dtype != MEO_F32 && t.param_dtype != MEO_BF16)
            return fail(MEO_EDTYPE, who + "param_dtype must be MEO_F32 or MEO_BF16");
        if (t.grad_dtype != MEO_F32 && t.grad_dtype != MEO_BF16)
            return fail(MEO_EDTYPE, who + "grad_dtype must be MEO_F32 or MEO_BF16");
        if (t.state_dtype != MEO_F32) return fail(MEO_EDTYPE, who + "GaLore states are float32 (state_dtype MEO_F32)");
        if (numel == 0) continue;
        if (!t.param) return fail(MEO_ENULL, who + "param is NULL");
        if (!t.grad) return fail(MEO_ENULL, who + "grad is NULL");
        if (reinterpret_cast<uintptr_t>(t.param) % (t.param_dtype == MEO_BF16 ? 2 : 4))
            return fail(MEO_EALIGN, who + "param misaligned for its dtype");
        if (reinterpret_cast<uintptr_t>(t.grad) % (t.grad_dtype == MEO_BF16 ? 2 : 4))
            return fail(MEO_EALIGN, who + "grad misaligned for its dtype");
        const meo_galore_state& s = st[k];
        if (!s.exp_avg) return fail(MEO_ENULL, who + "exp_avg is NULL");
        if (!s.exp_avg_sq) return fail(MEO_ENULL, who + "exp_avg_sq is NULL");
        if (reinterpret_cast<uintptr_t>(s.exp_avg) % 4 || reinterpret_cast<uintptr_t>(s.exp_avg_sq) % 4)
            return fail(MEO_EALIGN, who + "exp_avg or exp_avg_sq misaligned");
        if (ga_projected(t)) {
            if (t.grad_dtype != MEO_BF16)
                return fail(MEO_EDTYPE, who + "a projected (2-D) tensor needs a bf16 gradient");
            if (t.rows > kMaxDim || t.cols > kMaxDim) return fail(MEO_ESHAPE, who + "rows or cols exceed 2^31 - 1");
            const int32_t r = ga_rank(hp, t);
            if (r > kGaWide) return fail(MEO_EINVAL, who + "effective rank " + std::to_string(r) + " exceeds 256");
            if (!s.projector || !s.projector_t) return fail(MEO_ENULL, who + "projector or projector_t is NULL");
            if (reinterpret_cast<uintptr_t>(s.projector) % 2 || reinterpret_cast<uintptr_t>(s.projector_t) % 2)
                return fail(MEO_EALIGN, who + "projector misaligned");
            const int64_t D = ga_rows(hp, t);
            blocks[kGaProjR] += ceil_div(D, kGaTile);
            blocks[kGaBackR] += ceil_div(t.rows, kGaTile) * ceil_div(t.cols, kGaTile);
        } else {
            blocks[kGaFlat] += ceil_div(numel, kFlatTile);
        }
    }
    for (int64_t b : blocks)
        if (b > 0x7fffffffLL) return fail(MEO_ESHAPE, "the tensor list needs more than 2^31 blocks in one pass");
    return MEO_OK;
}

int check_galore_memory(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts, const meo_galore_state* st,
                        int dev) {
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        int64_t numel = 0;
        overflow_numel(t, &numel);
        if (numel == 0) continue;
        const std::string who = "tensor " + std::to_string(k) + ": ";
        const size_t ne = static_cast<size_t>(numel);
        const int32_t r = ga_rank(hp, t);
        const size_t mom = r ? static_cast<size_t>(ga_rows(hp, t)) * r : ne;
        struct Range { const void* p; size_t bytes; const char* name; };
        std::vector<Range> rs = {{t.param, ne * (t.param_dtype == MEO_BF16 ? 2 : 4), "param"},
                                 {t.grad, ne * (t.grad_dtype == MEO_BF16 ? 2 : 4), "grad"},
                                 {st[k].exp_avg, mom * 4, "exp_avg"}, {st[k].exp_avg_sq, mom * 4, "exp_avg_sq"}};
        if (r) {
            const size_t pu = static_cast<size_t>(ga_basis(hp, t)) * r * 2;
            rs.push_back({st[k].projector, pu, "projector"});
            rs.push_back({st[k].projector_t, pu, "projector_t"});
        }
        for (const Range& rg : rs) {
            const int rc = check_device_range(rg.p, rg.bytes, dev, who + rg.name, MEO_EMEMORY);
            if (rc) return rc;
        }
    }
    return MEO_OK;
}

int check_galore_workspace(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts, void* ws, size_t bytes) {
    const int64_t need = ga_layout(hp, n, ts, nullptr);
    if (need == 0) return MEO_OK;
    if (!ws) return fail(MEO_EWORKSPACE, "workspace is NULL");
    if (reinterpret_cast<uintptr_t>(ws) % 256) return fail(MEO_EWORKSPACE, "workspace not 256-byte aligned");
    if (bytes < static_cast<size_t>(need))
        return fail(MEO_EWORKSPACE, "workspace too small: need " + std::to_string(need) + " bytes");
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return fail(MEO_EHIP, "hipGetDevice failed");
    }
    return check_device_range(ws, bytes, dev, "workspace", MEO_EWORKSPACE);
}

GaPlan* get_galore_plan(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts, const meo_galore_state* st,
                        void* ws, int* rc) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        *rc = fail(MEO_EHIP, "hipGetDevice failed");
        return nullptr;
    }
    std::vector<uint8_t> key(sizeof(int) * 3 + sizeof(void*) + n * (sizeof(meo_tensor) + sizeof(meo_galore_state)));
    {
        uint8_t* w = key.data();
        const int hdr[3] = {n, dev, hp->rank * 2 + (hp->proj_type == MEO_GALORE_REVERSE_STD ? 1 : 0)};
        std::memcpy(w, hdr, sizeof hdr); w += sizeof hdr;
        std::memcpy(w, &ws, sizeof ws); w += sizeof ws;
        std::memcpy(w, ts, n * sizeof(meo_tensor)); w += n * sizeof(meo_tensor);
        std::memcpy(w, st, n * sizeof(meo_galore_state));
    }
    std::lock_guard<std::mutex> lock(g_mu);
    for (auto it = g_ga_plans.begin(); it != g_ga_plans.end(); ++it) {
        if ((*it)->key == key) {
            GaPlan* p = *it;
            g_ga_plans.erase(it);
            g_ga_plans.push_front(p);
            return p;
        }
    }
    *rc = check_galore_memory(hp, n, ts, st, dev);
    if (*rc) return nullptr;
    std::vector<int64_t> woff, roff;
    ga_layout(hp, n, ts, &woff, &roff);
    std::vector<RDesc> rd;
    std::vector<GDesc> right, left;
    std::vector<TDesc> flat;
    std::vector<int2> lists[kGaListCount];
    std::vector<int32_t> kr, kl;  // tensor indices of the right and left descriptors
    for (int32_t k = 0; k < n; ++k) {
        const meo_tensor& t = ts[k];
        int64_t numel = 0;
        overflow_numel(t, &numel);
        if (numel == 0) continue;
        const meo_galore_state& s = st[k];
        if (ga_projected(t)) {
            GDesc d;
            std::memset(&d, 0, sizeof d);
            d.m = static_cast<int32_t>(t.rows);
            d.n = static_cast<int32_t>(t.cols);
            const bool is_left = ga_left(hp, t);
            d.D = static_cast<int32_t>(ga_rows(hp, t));
            d.d = static_cast<int32_t>(ga_basis(hp, t));
            d.r = ga_rank(hp, t);
            d.g = static_cast<const uint16_t*>(t.grad);
            d.x = t.param;
            d.xbf16 = t.param_dtype == MEO_BF16;
            d.em = s.exp_avg;
            d.ev = s.exp_avg_sq;
            d.u = static_cast<uint16_t*>(s.projector);
            d.ut = static_cast<uint16_t*>(s.projector_t);
            uint8_t* wb = static_cast<uint8_t*>(ws) + woff[k];
            d.nh = reinterpret_cast<uint16_t*>(wb);
            d.nl = reinterpret_cast<uint16_t*>(wb + (static_cast<int64_t>(d.D) * d.r * 2 + 255) / 256 * 256);
            d.vec = aligned16(d.g) && aligned16(d.u) && aligned16(d.ut) && d.n % 8 == 0 && d.d % 8 == 0 &&
                    d.r % 8 == 0;
            d.rvec = aligned16(d.em) && aligned16(d.ev) && d.r % 8 == 0;
            d.wvec = aligned16(d.x) && d.n % 8 == 0;
            d.btj = static_cast<int32_t>(is_left ? ceil_div(d.n, kGaTile * kGaBackRW) : ceil_div(d.n, kGaWide));
            (is_left ? left : right).push_back(d);
            (is_left ? kl : kr).push_back(k);
            // refresh descriptor
            RDesc q;
            std::memset(&q, 0, sizeof q);
            q.g = d.g; q.u = d.u; q.ut = d.ut;
            q.m = d.m; q.n = d.n; q.D = d.D; q.d = d.d; q.r = d.r; q.p = d.r;
            q.left = is_left;
            q.gvec = aligned16(d.g) && d.n % 8 == 0;
            q.seed = k;
            uint8_t* rb = static_cast<uint8_t*>(ws) + roff[k];
            const int64_t sq = align256(static_cast<int64_t>(q.r) * q.d * 4);
            const int64_t sy = align256(static_cast<int64_t>(q.r) * std::max(q.D, q.d) * 4);
            const int64_t ss = align256(static_cast<int64_t>(q.r) * q.r * 8);
            q.qa = reinterpret_cast<float*>(rb);
            q.qb = reinterpret_cast<float*>(rb + sq);
            q.yt = reinterpret_cast<float*>(rb + 2 * sq);
            q.s = reinterpret_cast<double*>(rb + 2 * sq + sy);
            q.w = reinterpret_cast<double*>(rb + 2 * sq + sy + ss);
            q.s2 = reinterpret_cast<double*>(rb + 2 * sq + sy + 2 * ss);
            q.w2 = reinterpret_cast<double*>(rb + 2 * sq + sy + 3 * ss);
            const int id = static_cast<int>(rd.size());
            rd.push_back(q);
            auto addr = [&](int list, int64_t count) {
                for (int64_t i = 0; i < count; ++i) lists[list].push_back(make_int2(id, static_cast<int>(i)));
            };
            addr(kRfInit, ceil_div(static_cast<int64_t>(q.p) * q.d, kThreads * kVec));
            addr(is_left ? kRfG0T : kRfG0N, ceil_div(q.D, kGaTile));
            addr(is_left ? kRfG1N : kRfG1T, ceil_div(q.d, kGaTile));
            addr(kRfGram, ceil_div(q.p, 64) * ceil_div(q.p, 64));
            addr(kRfOne, 1);
            addr(kRfCols, ceil_div(q.p, 64) * ceil_div(q.d, 64));
            addr(kRfStore, q.r);
        } else {
            TDesc d;
            std::memset(&d, 0, sizeof d);
            d.x = t.param;
            d.g = t.grad;
            d.m = s.exp_avg;
            d.v = s.exp_avg_sq;
            d.numel = numel;
            d.gbf16 = t.grad_dtype == MEO_BF16;
            d.xbf16 = t.param_dtype == MEO_BF16;
            d.vec = aligned16(d.x) && aligned16(d.g) && aligned16(d.m) && aligned16(d.v);
            const int32_t id = static_cast<int32_t>(flat.size());
            flat.push_back(d);
            for (int64_t i = 0; i < ceil_div(numel, kFlatTile); ++i) lists[kGaFlat].push_back(make_int2(id, static_cast<int>(i)));
        }
    }
    // Back-projection kernel per side (see BackMode): the U-register kernel when every
    // rank is a multiple of kGaKb, rows allow 16-byte access and all parameters share
    // a dtype; its items cover 256 rows of U x up to kUrTiles tiles of N.
    int back_mode[2] = {kBackReg, kBackReg};
    for (int side = 0; side < 2; ++side) {
        const std::vector<GDesc>& v = side ? left : right;
        bool direct = true, all_f32 = true, all_bf16 = true;
        for (const GDesc& d : v) {
            direct = direct && d.vec && d.r % kGaKb == 0;
            all_f32 = all_f32 && !d.xbf16;
            all_bf16 = all_bf16 && d.xbf16;
        }
        back_mode[side] = !direct ? kBackReg : all_f32 ? kBackUr : all_bf16 ? kBackUrBf16 : kBackDirect;
    }
    for (int side = 0; side < 2; ++side)
        if (back_mode[side] == kBackUr || back_mode[side] == kBackUrBf16)
            for (GDesc& d : side ? left : right) d.btj = static_cast<int32_t>(ceil_div(ceil_div(d.D, kGaTile), kUrTiles));
    // Right descriptors first, then left; the item tables index that array.
    std::vector<GDesc> gd(right);
    gd.insert(gd.end(), left.begin(), left.end());
    bool proj_direct[2] = {true, true};  // right, left
    for (const GDesc& d : right) proj_direct[0] = proj_direct[0] && d.vec && d.d % kGaKb == 0;
    for (const GDesc& d : left) proj_direct[1] = proj_direct[1] && d.vec && d.d % kGaKb == 0;
    for (size_t i = 0; i < gd.size(); ++i) {
        const GDesc& d = gd[i];
        const bool is_left = i >= right.size();
        const int id = static_cast<int>(i);
        const int64_t pt = ceil_div(d.D, proj_direct[is_left] ? kGaPwRows : kGaProjRows);
        // both sides direct: one list (kGaProjR) for the mixed kernel
        const bool one_list = proj_direct[0] && proj_direct[1];
        for (int64_t y = 0; y < pt; ++y)
            lists[is_left && !one_list ? kGaProjL : kGaProjR].push_back(make_int2(id, static_cast<int>(y)));
        std::vector<int2>& L = lists[is_left ? kGaBackL : kGaBackR];
        if (back_mode[is_left] == kBackUr || back_mode[is_left] == kBackUrBf16) {
            // chunks of N outer, bands of U inner: consecutive items share N's rows
            const int64_t bands = ceil_div(d.d, kGaWide);
            for (int64_t c = 0; c < d.btj; ++c)
                for (int64_t b = 0; b < bands; ++b) L.push_back(make_int2(id, static_cast<int>(b * d.btj + c)));
            continue;
        }
        // Back-projection tiles, tile rows of N outer and tiles of U inner, so
        // that consecutive blocks share a tile of N; xcd_deal below then puts the
        // whole tensor on one XCD.
        const int64_t ti_n = is_left ? ceil_div(d.m, kGaWide) : ceil_div(d.m, kGaTile * kGaBackRW);
        const int64_t na = is_left ? d.btj : ti_n;   // tiles of N
        const int64_t nb = is_left ? ti_n : d.btj;   // tiles of U
        for (int64_t a = 0; a < na; ++a)
            for (int64_t b = 0; b < nb; ++b) {
                const int64_t ti = is_left ? b : a, tj = is_left ? a : b;
                L.push_back(make_int2(id, static_cast<int>(ti * d.btj + tj)));
            }
    }
    // Every tile of a tensor on one XCD: its L2 then fetches the tensor's projector
    // and low-rank arrays once (measured on the 7B list: projection -0.8%,
    // back-projection -2.4%).
    xcd_deal(lists[kGaProjR]);
    xcd_deal(lists[kGaProjL]);
    xcd_deal(lists[kGaBackR]);
    xcd_deal(lists[kGaBackL]);
    size_t offs[kGaListCount];
    size_t total = (gd.size() * sizeof(GDesc) + 255) / 256 * 256;
    const size_t foff = total;
    total += (flat.size() * sizeof(TDesc) + 255) / 256 * 256;
    const size_t roffb = total;
    total += (rd.size() * sizeof(RDesc) + 255) / 256 * 256;
    for (int l = 0; l < kGaListCount; ++l) {
        offs[l] = total;
        total += (lists[l].size() * sizeof(int2) + 255) / 256 * 256;
    }
    total = std::max<size_t>(total, 256);
    std::vector<uint8_t> host(total, 0);
    if (!gd.empty()) std::memcpy(host.data(), gd.data(), gd.size() * sizeof(GDesc));
    if (!flat.empty()) std::memcpy(host.data() + foff, flat.data(), flat.size() * sizeof(TDesc));
    if (!rd.empty()) std::memcpy(host.data() + roffb, rd.data(), rd.size() * sizeof(RDesc));
    for (int l = 0; l < kGaListCount; ++l)
        if (!lists[l].empty()) std::memcpy(host.data() + offs[l], lists[l].data(), lists[l].size() * sizeof(int2));
    GaPlan* p = new GaPlan;
    p->key = std::move(key);
    p->device = dev;
    p->back_mode[0] = back_mode[0];
    p->back_mode[1] = back_mode[1];
    p->proj_direct[0] = proj_direct[0];
    p->proj_direct[1] = proj_direct[1];
    p->nright = static_cast<int>(right.size());
    if (hipMalloc(&p->mem, host.size()) != hipSuccess ||
        hipMemcpy(p->mem, host.data(), host.size(), hipMemcpyHostToDevice) != hipSuccess) {
        if (p->mem) (void)hipFree(p->mem);
        delete p;
        *rc = fail(MEO_EHIP, "could not allocate or upload the launch table");
        return nullptr;
    }
    uint8_t* base = static_cast<uint8_t*>(p->mem);
    p->gdesc = reinterpret_cast<const GDesc*>(base);
    p->fdesc = reinterpret_cast<const TDesc*>(base + foff);
    p->rdesc = reinterpret_cast<const RDesc*>(base + roffb);
    for (int l = 0; l < kGaListCount; ++l) {
        p->items[l] = reinterpret_cast<const int2*>(base + offs[l]);
        p->count[l] = static_cast<int64_t>(lists[l].size());
    }
    g_ga_plans.push_front(p);
    while (g_ga_plans.size() > kMaxPlans) {
        GaPlan* q = g_ga_plans.back();
        g_ga_plans.pop_back();
        (void)hipFree(q->mem);
        delete q;
    }
    return p;
}

}  // namespace

void meo_galore_defaults(meo_galore_hparams* hp) {
    if (!hp) return;
    std::memset(hp, 0, sizeof *hp);
    hp->lr = 1e-3;
    hp->beta1 = 0.9;
    hp->beta2 = 0.999;
    hp->eps = 1e-8;
    hp->weight_decay = 0.0;
    hp->rank = 256;
    hp->update_proj_gap = 200;
    hp->scale = 0.25;
    hp->proj_type = MEO_GALORE_STD;
}

int32_t meo_galore_rank(const meo_galore_hparams* hp, const meo_tensor* t) {
    if (!hp || !t || hp->rank < 1) return 0;
    return ga_rank(hp, *t);
}

size_t meo_galore_workspace_size(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts) {
    if (!hp || n <= 0 || !ts || hp->rank < 1) return 0;
    return static_cast<size_t>(ga_layout(hp, n, ts, nullptr));
}

int meo_galore_validate(const meo_galore_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                        const meo_galore_state* st) {
    g_err.clear();
    const int rc = check_galore_hp(hp);
    if (rc) return rc;
    return check_galore_tensors(hp, step, n, ts, st);
}

int meo_galore_refresh(const meo_galore_hparams* hp, int32_t n, const meo_tensor* ts, const meo_galore_state* st,
                       void* ws, size_t ws_bytes, void* stream) {
    int rc = meo_galore_validate(hp, 1, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_galore_workspace(hp, n, ts, ws, ws_bytes);
    if (rc) return rc;
    GaPlan* p = get_galore_plan(hp, n, ts, st, ws, &rc);
    if (!p) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    auto tab = [&](int l) { return RTable{p->rdesc, p->items[l]}; };
    auto cnt = [&](int l) { return p->count[l]; };
    if (cnt(kRfOne) == 0) return MEO_OK;
    PassTimer pt(s);
    // Cholesky-QR of the p x d block in `src`, into `dst`.
    auto cholqr = [&](int src, int dst) {
        launch_rf_gram(tab(kRfGram), cnt(kRfGram), src, false, s);
        launch_rf_chol(tab(kRfOne), cnt(kRfOne), s);
        launch_rf_trmm(tab(kRfCols), cnt(kRfCols), src, dst, s);
    };
    // Twice, for rows orthonormal to fp32 rounding (the start block and the block
    // of the Rayleigh-Ritz step); once between products, where a well-conditioned
    // basis is enough. The result ends in `buf`.
    auto cholqr2 = [&](int buf) {
        const int other = buf == kRbQa ? kRbQb : kRbQa;
        cholqr(buf, other);
        cholqr(other, buf);
    };
    auto times_xt = [&](int src, int dst) {  // Y^T = Q^T X^T
        launch_rf_gemm(tab(kRfG0N), cnt(kRfG0N), 0, src, dst, false, s);
        launch_rf_gemm(tab(kRfG0T), cnt(kRfG0T), 0, src, dst, true, s);
    };
    launch_rf_init(tab(kRfInit), cnt(kRfInit), kRbQa, s);
    cholqr2(kRbQa);
    for (int i = 0; i < kRfIters; ++i) {
        times_xt(kRbQa, kRbYt);
        launch_rf_gemm(tab(kRfG1N), cnt(kRfG1N), 1, kRbYt, kRbQb, false, s);  // Z^T = Y^T X
        launch_rf_gemm(tab(kRfG1T), cnt(kRfG1T), 1, kRbYt, kRbQb, true, s);
        if (i + 1 < kRfIters) {
            cholqr(kRbQb, kRbQa);
        } else {
            cholqr(kRbQb, kRbQa);
            cholqr2(kRbQa);
        }
    }
    times_xt(kRbQa, kRbYt);
    launch_rf_gram(tab(kRfGram), cnt(kRfGram), kRbYt, true, s);
    launch_rf_jacobi(tab(kRfOne), cnt(kRfOne), s);
    launch_rf_basis(tab(kRfCols), cnt(kRfCols), kRbQa, s);
    launch_rf_store(tab(kRfStore), cnt(kRfStore), s);
    pt.mark(kPassGaRefresh);
    return launch_status("galore refresh launch");
}

int meo_galore_step(const meo_galore_hparams* hp, int64_t step, int32_t n, const meo_tensor* ts,
                    const meo_galore_state* st, void* ws, size_t ws_bytes, void* stream) {
    int rc = meo_galore_validate(hp, step, n, ts, st);
    if (rc) return rc;
    if (n == 0) return MEO_OK;
    rc = check_galore_workspace(hp, n, ts, ws, ws_bytes);
    if (rc) return rc;
    if ((step - 1) % hp->update_proj_gap == 0) {
        rc = meo_galore_refresh(hp, n, ts, st, ws, ws_bytes, stream);
        if (rc) return rc;
    }
    GaPlan* p = get_galore_plan(hp, n, ts, st, ws, &rc);
    if (!p) return rc;
    const hipStream_t s = static_cast<hipStream_t>(stream);
    const double tt = static_cast<double>(step);
    const double bc1 = 1.0 - std::pow(hp->beta1, tt), bc2 = 1.0 - std::pow(hp->beta2, tt);
    GaArgs a{static_cast<float>(hp->beta1), static_cast<float>(hp->beta2), static_cast<float>(1.0 - hp->beta1),
             static_cast<float>(1.0 - hp->beta2), static_cast<float>(1.0 / bc1), static_cast<float>(1.0 / bc2),
             static_cast<float>(hp->eps), static_cast<float>(1.0 - hp->lr * hp->weight_decay),
             static_cast<float>(hp->lr * hp->scale)};
    PassTimer pt(s);
    if (p->proj_direct[0] && p->proj_direct[1]) {
        launch_galore_project_mixed(GTable{p->gdesc, p->items[kGaProjR]}, p->count[kGaProjR], p->nright, a, s);
    } else {
        launch_galore_project(GTable{p->gdesc, p->items[kGaProjR]}, p->count[kGaProjR], a, false, p->proj_direct[0], s);
        launch_galore_project(GTable{p->gdesc, p->items[kGaProjL]}, p->count[kGaProjL], a, true, p->proj_direct[1], s);
    }
    pt.mark(kPassGaProject);
    launch_galore_back(GTable{p->gdesc, p->items[kGaBackR]}, p->count[kGaBackR], a, false, p->back_mode[0], s);
    launch_galore_back(GTable{p->gdesc, p->items[kGaBackL]}, p->count[kGaBackL], a, true, p->back_mode[1], s);
    pt.mark(kPassGaBack);
    a.coef = static_cast<float>(hp->lr);
    launch_galore_adamw(Table{p->fdesc, p->items[kGaFlat], nullptr}, p->count[kGaFlat], a, s);
    pt.mark(kPassGaAdamw);
    return launch_status("galore step launch");
}

}  // extern "C"
