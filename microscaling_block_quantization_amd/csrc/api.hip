// api.hip -- the extern "C" entry points of libmx.so (declared in include/mx.h):
// argument validation, buffer-size queries and kernel dispatch.  Every check
// happens before the first launch; the library allocates nothing.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include "../../include/mx.h"
#include "mx_kernels.hpp"

using mxk::QParams;

namespace {

constexpr size_t ALIGN = 256;

size_t round_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Validate a format for a rows x cols tensor.  Returns MX_OK or an error code.
int check_format(const mx_format* f, int64_t rows, int64_t cols) {
    if (!f) return MX_ERR_ARG;
    if (f->elem < 0 || f->elem > MX_ELEM_FP8_E5M2) return MX_ERR_ARG;
    if (f->scale < 0 || f->scale > MX_SCALE_E3M0) return MX_ERR_ARG;
    if (f->rule < 0 || f->rule > MX_RULE_OAS) return MX_ERR_ARG;
    if (f->round < 0 || f->round > MX_ROUND_CEIL) return MX_ERR_ARG;
    if (f->asymmetric != 0 && f->asymmetric != 1) return MX_ERR_ARG;
    if (rows < 0 || cols < 0) return MX_ERR_ARG;
    const int br = f->block_rows, bc = f->block_cols;
    if (br < 1 || bc < 1 || !is_pow2(br) || !is_pow2(bc)) return MX_ERR_ARG;
    if (rows % br || cols % bc) return MX_ERR_ARG;
    if (br == 1) {
        if (bc < 8 || bc > 256) return MX_ERR_UNSUPPORTED;
    } else {
        if (br < 8 || br > 32) return MX_ERR_UNSUPPORTED;
        if (bc != 1 && bc != br) return MX_ERR_UNSUPPORTED;
    }
    if (cols % 8) return MX_ERR_UNSUPPORTED;
    const mxd::Elem E = mxd::make_elem(f->elem, f->asymmetric);
    if (f->asymmetric) {
        if (f->elem != MX_ELEM_E2M1 && f->elem != MX_ELEM_INT4) return MX_ERR_UNSUPPORTED;
        if (f->scale != MX_SCALE_E8M0 || f->hadamard || f->macro_cols) return MX_ERR_UNSUPPORTED;
    }
    if (f->rule == MX_RULE_OAS && (f->scale == MX_SCALE_E8M0 || f->macro_cols)) {
        if (!(f->oas_tau >= E.qmax && f->oas_tau < 2.0f * E.qmax)) return MX_ERR_ARG;
    }
    if (f->hadamard) {
        const int h = f->hadamard;
        if (h != 16 && h != 32 && h != 64 && h != 128) return MX_ERR_UNSUPPORTED;
        if (br != 1 || cols % h) return MX_ERR_UNSUPPORTED;
    }
    if (f->macro_cols) {
        if (f->macro_cols != 128) return MX_ERR_ARG;
        if (br != 1 || 128 % bc || cols % 128 || f->scale != MX_SCALE_E8M0) return MX_ERR_UNSUPPORTED;
    }
    return MX_OK;
}

int64_t crow_bytes(const mx_format* f, int64_t cols) {
    return mxd::code_row_bytes(mxd::make_elem(f->elem, f->asymmetric).bits, cols);
}

QParams make_params(const mx_format* f, int in_bf16, const void* x, int64_t rows, int64_t cols, int64_t ld,
                    const mx_qtensor* q) {
    QParams p;
    memset(&p, 0, sizeof(p));
    p.x = x;
    p.rows = rows;
    p.cols = cols;
    p.ld = ld;
    p.in_bf16 = in_bf16;
    p.codes = static_cast<uint8_t*>(q->codes);
    p.scales = static_cast<uint8_t*>(q->scales);
    p.offsets = static_cast<uint16_t*>(q->offsets);
    p.macro = static_cast<uint8_t*>(q->macro_scales);
    p.tensor_scale = q->tensor_scale;
    p.ref_exp = q->ref_exp;
    p.elem = f->elem;
    p.asym = f->asymmetric;
    p.scale = f->scale;
    p.rule = f->rule;
    p.round = f->round;
    p.br = f->block_rows;
    p.bc = f->block_cols;
    p.had = f->hadamard;
    p.macro_cols = f->macro_cols;
    p.tau = f->oas_tau;
    p.seed = f->seed;
    p.off = f->rng_offset;
    return p;
}

bool needs_prepass(const mx_format* f) { return f->scale == MX_SCALE_NVFP4 || f->scale == MX_SCALE_E3M0; }

// workgroups of the quantization kernel this call launches (its statistics
// partials: one per workgroup)
int64_t quant_grid(const QParams& p) {
    if (p.br > 1) return mxk::tiles_grid(p);
    if (mxk::rows_fast_ok(p)) return mxk::rows_fast_grid(p);
    if (mxk::rows_fp8_ok(p)) return mxk::rows_fp8_grid(p);
    if (mxk::rows_fp6_ok(p)) return mxk::rows_fp6_grid(p);
    if (mxk::rows_hw_ok(p)) return mxk::rows_hw_grid(p);
    return mxk::rows_grid(p);
}

// the largest grid any call with this format and shape can launch, whatever
// the input dtype, the dequant output and the row stride: a strided input
// moves a dense-row format from the fast or wave-tile kernel (grid capped) to
// the general row kernel (one workgroup per 256 chunks)
int64_t max_quant_grid(QParams p) {
    int64_t g = 0;
    for (int bf = 0; bf < 2; bf++) {
        p.in_bf16 = bf;
        if (p.br > 1) {
            g = std::max(g, mxk::tiles_grid(p));
            continue;
        }
        g = std::max(g, mxk::rows_grid(p));
        p.dq = nullptr;
        p.ld = p.cols;
        if (mxk::rows_fast_ok(p)) g = std::max(g, mxk::rows_fast_grid(p));
        if (mxk::rows_fp8_ok(p)) g = std::max(g, mxk::rows_fp8_grid(p));
        if (mxk::rows_fp6_ok(p)) g = std::max(g, mxk::rows_fp6_grid(p));
        if (mxk::rows_hw_ok(p)) g = std::max(g, mxk::rows_hw_grid(p));
    }
    return g;
}

struct Workspace {
    size_t stats_off, stats_bytes, amax_off, amax_bytes, total;
};

// One layout per format and shape, valid for both input dtypes and every
// kernel route, so that mx_query_sizes needs neither.
Workspace workspace_layout(const mx_format* f, int64_t rows, int64_t cols) {
    mx_qtensor dummy;
    memset(&dummy, 0, sizeof(dummy));
    QParams p = make_params(f, 1, nullptr, rows, cols, cols, &dummy);
    Workspace w;
    w.stats_off = 0;
    w.stats_bytes = round_up((size_t)max_quant_grid(p) * sizeof(mxd::StatPart));
    w.amax_off = w.stats_off + w.stats_bytes;
    int64_t ga = 0;
    for (int bf = 0; bf < 2; bf++) {
        p.in_bf16 = bf;
        ga = std::max(ga, mxk::amax_grid(p));
    }
    w.amax_bytes = needs_prepass(f) ? round_up((size_t)ga * sizeof(float)) : 0;
    w.total = w.amax_off + w.amax_bytes;
    return w;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MX_OK : MX_ERR_HIP; }

// Every check of mx_quantize except the workspace's.
int check_quantize(const mx_format* f, int in_dtype, const void* x, int64_t rows, int64_t cols, int64_t ld,
                   const mx_qtensor* out, const void* dequant, int dq_dtype, const mx_stats* stats) {
    int rc = check_format(f, rows, cols);
    if (rc) return rc;
    if (in_dtype != MX_DTYPE_F32 && in_dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
    if (dequant && dq_dtype != MX_DTYPE_F32 && dq_dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
    if (!out || ld < cols) return MX_ERR_ARG;
    const int64_t n = rows * cols;
    if (n > 0 && (!x || !out->codes || !out->scales)) return MX_ERR_ARG;
    if (f->asymmetric && n > 0 && !out->offsets) return MX_ERR_ARG;
    if (f->macro_cols && n > 0 && !out->macro_scales) return MX_ERR_ARG;
    if (f->scale == MX_SCALE_NVFP4 && !out->tensor_scale) return MX_ERR_ARG;
    if (f->scale == MX_SCALE_E3M0 && !out->ref_exp) return MX_ERR_ARG;
    const int esz = in_dtype == MX_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(x) || !aligned16(out->codes) || !aligned16(dequant) || ((ld * esz) & 15)) return MX_ERR_ALIGN;
    if (!aligned16(out->offsets) || !aligned16(stats)) return MX_ERR_ALIGN;
    return MX_OK;
}

// The launches of one quantization, its arguments already checked.  ws: the
// workspace laid out as W (unused, and may be null, when the call needs none).
int launch_quantize(const mx_format* f, int in_dtype, const void* x, int64_t rows, int64_t cols, int64_t ld,
                    const mx_qtensor* out, void* dequant, int dq_dtype, mx_stats* stats, uint8_t* ws,
                    const Workspace& W, hipStream_t s) {
    int rc;
    const int64_t n = rows * cols;
    QParams p = make_params(f, in_dtype == MX_DTYPE_BF16, x, rows, cols, ld, out);
    p.dq = dequant;
    p.dq_bf16 = dq_dtype == MX_DTYPE_BF16;

    if (needs_prepass(f)) {
        QParams a = p;
        a.amax_parts = reinterpret_cast<float*>(ws + W.amax_off);
        int64_t ga = 0;
        if (n > 0) {
            rc = hip_status(mxk::launch_amax(a, s, &ga));
            if (rc) return rc;
        }
        const mxd::Elem E = mxd::make_elem(f->elem, f->asymmetric);
        rc = hip_status(mxk::launch_tensor_scale(a.amax_parts, ga, f->scale, E.qmax, out->tensor_scale,
                                                 out->ref_exp, s));
        if (rc) return rc;
    }
    int64_t grid = n > 0 ? quant_grid(p) : 0;
    if (stats) {
        // the layout covers every route; this guards the route taken
        if ((size_t)grid * sizeof(mxd::StatPart) > W.stats_bytes) return MX_ERR_WORKSPACE;
        p.parts = reinterpret_cast<mxd::StatPart*>(ws + W.stats_off);
    }
    if (grid > 0) {
        hipError_t e;
        if (p.br > 1) e = mxk::launch_tiles(p, s);
        else if (mxk::rows_fast_ok(p)) e = mxk::launch_rows_fast(p, s, &grid);
        else if (mxk::rows_fp8_ok(p)) e = mxk::launch_rows_fp8(p, s, &grid);
        else if (mxk::rows_fp6_ok(p)) e = mxk::launch_rows_fp6(p, s, &grid);
        else if (mxk::rows_hw_ok(p)) e = mxk::launch_rows_hw(p, s, &grid);
        else e = mxk::launch_rows(p, false, s);
        rc = hip_status(e);
        if (rc) return rc;
    }
    if (stats) {
        rc = hip_status(mxk::launch_stats_final(p.parts, grid, n, stats, s));
        if (rc) return rc;
    }
    return MX_OK;
}

// ---- the static scratch of mx_quantize_noalloc -----------------------------
// One copy per GPU, held until the process ends.  Host code never passes the
// array's name to a kernel (on the host it only names the symbol): it takes
// the device address hipGetSymbolAddress gives on each device, once per
// device, and passes that.
__device__ __align__(256) uint8_t scratch[MX_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::atomic<uint8_t*> scratch_ptr[MAX_DEVICES];

// The current device's address of `scratch`.
int static_scratch(uint8_t** ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return MX_ERR_HIP;
    uint8_t* p = scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return MX_ERR_HIP;
        p = static_cast<uint8_t*>(a);
        scratch_ptr[dev].store(p, std::memory_order_release);   // the same address if two threads race here
    }
    *ptr = p;
    return MX_OK;
}

}  // namespace

extern "C" {

const char* mx_status_string(int status) {
    switch (status) {
    case MX_OK: return "ok";
    case MX_ERR_ARG: return "invalid argument";
    case MX_ERR_UNSUPPORTED: return "format or shape not supported by this library";
    case MX_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case MX_ERR_WORKSPACE: return "workspace missing or too small";
    case MX_ERR_HIP: return "HIP launch failed";
    case MX_ERR_TOO_LARGE: return "tensor needs more scratch than mx_quantize_noalloc's static array holds";
    default: return "unknown status";
    }
}

int mx_query_sizes(const mx_format* f, int64_t rows, int64_t cols, mx_sizes* out) {
    int rc = check_format(f, rows, cols);
    if (rc) return rc;
    if (!out) return MX_ERR_ARG;
    const int64_t nblk = (rows / f->block_rows) * (cols / f->block_cols);
    out->codes = (size_t)(rows * crow_bytes(f, cols));
    out->scales = (size_t)nblk;
    out->offsets = f->asymmetric ? (size_t)nblk * 2 : 0;
    out->macro_scales = f->macro_cols ? (size_t)(rows * (cols / 128)) : 0;
    out->tensor_scale = f->scale == MX_SCALE_NVFP4 ? sizeof(float) : 0;
    out->ref_exp = f->scale == MX_SCALE_E3M0 ? sizeof(int32_t) : 0;
    out->workspace = workspace_layout(f, rows, cols).total;
    return MX_OK;
}

int mx_quantize(const mx_format* f, int in_dtype, const void* x, int64_t rows, int64_t cols, int64_t ld,
                const mx_qtensor* out, void* dequant, int dq_dtype, mx_stats* stats, void* workspace,
                size_t ws_bytes, void* stream) {
    int rc = check_quantize(f, in_dtype, x, rows, cols, ld, out, dequant, dq_dtype, stats);
    if (rc) return rc;
    const Workspace W = workspace_layout(f, rows, cols);
    const bool need_ws = stats || needs_prepass(f);
    if (need_ws && (!workspace || ws_bytes < W.total)) return MX_ERR_WORKSPACE;
    if (need_ws && !aligned16(workspace)) return MX_ERR_ALIGN;
    return launch_quantize(f, in_dtype, x, rows, cols, ld, out, dequant, dq_dtype, stats,
                           static_cast<uint8_t*>(workspace), W, static_cast<hipStream_t>(stream));
}

int mx_quantize_noalloc(const mx_format* f, int in_dtype, const void* x, int64_t rows, int64_t cols, int64_t ld,
                        const mx_qtensor* out, void* dequant, int dq_dtype, mx_stats* stats, void* stream) {
    int rc = check_quantize(f, in_dtype, x, rows, cols, ld, out, dequant, dq_dtype, stats);
    if (rc) return rc;
    const Workspace W = workspace_layout(f, rows, cols);
    const bool need_ws = stats || needs_prepass(f);
    if (need_ws && W.total > MX_NOALLOC_SCRATCH_BYTES) return MX_ERR_TOO_LARGE;
    uint8_t* ws = nullptr;
    if (need_ws) {
        rc = static_scratch(&ws);
        if (rc) return rc;
    }
    return launch_quantize(f, in_dtype, x, rows, cols, ld, out, dequant, dq_dtype, stats, ws, W,
                           static_cast<hipStream_t>(stream));
}

int mx_quantize_many(const mx_format* f, int in_dtype, const mx_qjob* jobs, int count, void* stream) {
    if (count < 0 || (count > 0 && !jobs)) return MX_ERR_ARG;
    if (count == 0) {
        if (in_dtype != MX_DTYPE_F32 && in_dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
        return check_format(f, 0, 0);
    }
    // every check before the first launch
    for (int i = 0; i < count; i++) {
        const mx_qjob& J = jobs[i];
        int rc = check_quantize(f, in_dtype, J.x, J.rows, J.cols, J.ld, J.out, nullptr, 0, J.stats);
        if (rc) return rc;
        const bool need_ws = J.stats || needs_prepass(f);
        if (!need_ws) continue;
        const size_t used = workspace_layout(f, J.rows, J.cols).total;
        if (!J.workspace || J.ws_bytes < used) return MX_ERR_WORKSPACE;
        if (!aligned16(J.workspace)) return MX_ERR_ALIGN;
        // jobs may run at the same time: their workspaces must not overlap
        const uintptr_t lo = (uintptr_t)J.workspace, hi = lo + used;
        for (int k = 0; k < i; k++) {
            const mx_qjob& O = jobs[k];
            if (!(O.stats || needs_prepass(f))) continue;
            const uintptr_t olo = (uintptr_t)O.workspace, ohi = olo + workspace_layout(f, O.rows, O.cols).total;
            if (lo < ohi && olo < hi) return MX_ERR_ARG;
        }
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int bf = in_dtype == MX_DTYPE_BF16;
    // dense MXFP4-style rows: up to MANY_MAX jobs per launch, jobs with
    // statistics and jobs without in separate launches (the statistics are a
    // compile-time variant of the kernel)
    auto shared = [&](const mx_qjob& J) {
        if (J.rows * J.cols == 0) return false;
        QParams p = make_params(f, bf, J.x, J.rows, J.cols, J.ld, J.out);
        return mxk::rows_fast_ok(p);
    };
    for (int st = 0; st < 2; st++) {
        mxk::FastMany m;
        memset(&m, 0, sizeof(m));
        int idx[mxk::MANY_MAX];
        auto flush = [&]() -> int {
            if (m.count == 0) return MX_OK;
            const mx_qjob& J0 = jobs[idx[0]];
            QParams p = make_params(f, bf, J0.x, J0.rows, J0.cols, J0.ld, J0.out);
            p.parts = st ? m.job[0].parts : nullptr;
            int64_t grid = 0;
            int rc = hip_status(mxk::launch_rows_fast_many(p, m, s, &grid));
            if (rc) return rc;
            if (st) {
                // each job's nb is at most its tensor's rows_fast_grid, which its
                // workspace layout holds
                mxk::FinalMany fm;
                for (int k = 0; k < m.count; k++) {
                    const mx_qjob& J = jobs[idx[k]];
                    fm.job[k] = mxk::FinalJob{m.job[k].parts, m.job[k].nb, J.rows * J.cols, J.stats};
                }
                rc = hip_status(mxk::launch_stats_final_many(fm, m.count, s));
                if (rc) return rc;
            }
            m.count = 0;
            return MX_OK;
        };
        for (int i = 0; i < count; i++) {
            const mx_qjob& J = jobs[i];
            if ((J.stats != nullptr) != (st == 1) || !shared(J)) continue;
            mxk::FastJob& F = m.job[m.count];
            F.x = J.x;
            F.codes = static_cast<uint8_t*>(J.out->codes);
            F.scales = static_cast<uint8_t*>(J.out->scales);
            F.parts = st ? reinterpret_cast<mxd::StatPart*>(static_cast<uint8_t*>(J.workspace) +
                                                            workspace_layout(f, J.rows, J.cols).stats_off)
                         : nullptr;
            F.nchunks = J.rows * J.cols / (bf ? 8 : 4);
            idx[m.count++] = i;
            if (m.count == mxk::MANY_MAX) {
                const int rc = flush();
                if (rc) return rc;
            }
        }
        const int rc = flush();
        if (rc) return rc;
    }
    // every other job on its own
    for (int i = 0; i < count; i++) {
        const mx_qjob& J = jobs[i];
        if (shared(J)) continue;
        const int rc = launch_quantize(f, in_dtype, J.x, J.rows, J.cols, J.ld, J.out, nullptr, 0, J.stats,
                                       static_cast<uint8_t*>(J.workspace), workspace_layout(f, J.rows, J.cols), s);
        if (rc) return rc;
    }
    return MX_OK;
}

int mx_dequantize(const mx_format* f, const mx_qtensor* q, int out_dtype, void* y, int64_t ld, void* stream) {
    if (!q) return MX_ERR_ARG;
    int rc = check_format(f, q->rows, q->cols);
    if (rc) return rc;
    if (out_dtype != MX_DTYPE_F32 && out_dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
    if (ld < q->cols) return MX_ERR_ARG;
    const int64_t n = q->rows * q->cols;
    if (n == 0) return MX_OK;
    if (!y || !q->codes || !q->scales) return MX_ERR_ARG;
    if (f->asymmetric && !q->offsets) return MX_ERR_ARG;
    if (f->macro_cols && !q->macro_scales) return MX_ERR_ARG;
    if (f->scale == MX_SCALE_NVFP4 && !q->tensor_scale) return MX_ERR_ARG;
    if (f->scale == MX_SCALE_E3M0 && !q->ref_exp) return MX_ERR_ARG;
    const int esz = out_dtype == MX_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(y) || !aligned16(q->codes) || ((ld * esz) & 15)) return MX_ERR_ALIGN;
    QParams p = make_params(f, 0, nullptr, q->rows, q->cols, ld, q);
    p.dq = y;
    p.dq_bf16 = out_dtype == MX_DTYPE_BF16;
    return hip_status(mxk::launch_dequant(p, static_cast<hipStream_t>(stream)));
}

size_t mx_qsnr_workspace_size(int64_t n) {
    if (n < 0) return 0;
    return round_up((size_t)mxk::qsnr_grid(n) * sizeof(mxd::StatPart)) + round_up(sizeof(mx_stats));
}

int mx_qsnr(int dtype, const void* ref, const void* approx, int64_t n, mx_stats* host_stats, double* qsnr_db,
            void* workspace, size_t ws_bytes, void* stream) {
    if (dtype != MX_DTYPE_F32 && dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
    if (n <= 0 || !ref || !approx || !qsnr_db) return MX_ERR_ARG;
    if (!aligned16(ref) || !aligned16(approx)) return MX_ERR_ALIGN;
    const size_t need = mx_qsnr_workspace_size(n);
    if (!workspace || ws_bytes < need) return MX_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MX_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    mxd::StatPart* parts = reinterpret_cast<mxd::StatPart*>(ws);
    void* fin = ws + round_up((size_t)mxk::qsnr_grid(n) * sizeof(mxd::StatPart));
    int rc = hip_status(mxk::launch_qsnr(dtype == MX_DTYPE_BF16, ref, approx, n, parts, s));
    if (rc) return rc;
    rc = hip_status(mxk::launch_stats_final(parts, mxk::qsnr_grid(n), n, fin, s));
    if (rc) return rc;
    mx_stats st;
    if (hipMemcpyAsync(&st, fin, sizeof(st), hipMemcpyDeviceToHost, s) != hipSuccess) return MX_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return MX_ERR_HIP;
    if (host_stats) *host_stats = st;
    if (!(st.sig2 > 0)) return MX_ERR_ARG;
    *qsnr_db = st.err2 > 0 ? 10.0 * log10(st.sig2 / st.err2) : INFINITY;
    return MX_OK;
}

int mx_gemm(const mx_format* fa, const mx_qtensor* a, const mx_format* fb, const mx_qtensor* b, void* c,
            int64_t ldc, int c_dtype, void* stream) {
    if (!fa || !fb || !a || !b) return MX_ERR_ARG;
    for (const mx_format* f : {fa, fb})
        if (f->block_rows != 1 || f->asymmetric || f->hadamard) return MX_ERR_UNSUPPORTED;
    // E8M0 scales on 1 x 32 blocks (MX): the scaled matrix instruction, any
    // element pair of E2M1 / E2M3 / E3M2, macro scales allowed on MXFP4
    const bool native = fa->scale == MX_SCALE_E8M0 && fb->scale == MX_SCALE_E8M0 && fa->block_cols == 32 &&
                        fb->block_cols == 32 && mxk::gemm_elem_ok(fa->elem) && mxk::gemm_elem_ok(fb->elem);
    if (!native) {
        // E2M1 under E8M0, UE4M3, NVFP4 or UE5M3 scales on any row block:
        // decoded to bf16 for the bf16 matrix instruction.  Macro-block scales
        // (MBS over E8M0 sub-blocks of other widths than 32, e.g. 1 x 16) fold
        // into the decode; both operands then carry E8M0 block scales.
        for (const mx_format* f : {fa, fb})
            if (f->elem != MX_ELEM_E2M1 || !mxk::gemm_upcvt_scale_ok(f->scale)) return MX_ERR_UNSUPPORTED;
        if ((fa->macro_cols || fb->macro_cols) && (fa->scale != MX_SCALE_E8M0 || fb->scale != MX_SCALE_E8M0))
            return MX_ERR_UNSUPPORTED;
    }
    // macro-block scales: E2M1 operands only (on the native route the
    // sub-blocks are the 1 x 32 blocks the instruction scales)
    const bool mbs = fa->macro_cols || fb->macro_cols;
    if (mbs && (fa->elem != MX_ELEM_E2M1 || fb->elem != MX_ELEM_E2M1)) return MX_ERR_UNSUPPORTED;
    int rc = check_format(fa, a->rows, a->cols);
    if (rc) return rc;
    rc = check_format(fb, b->rows, b->cols);
    if (rc) return rc;
    const int64_t M = a->rows, N = b->rows, K = a->cols;
    if (b->cols != K) return MX_ERR_ARG;
    if (c_dtype != MX_DTYPE_F32 && c_dtype != MX_DTYPE_BF16) return MX_ERR_ARG;
    if (K % 32) return MX_ERR_UNSUPPORTED;
    if (ldc < N) return MX_ERR_ARG;
    if (M == 0 || N == 0) return MX_OK;
    if (K == 0) return MX_ERR_UNSUPPORTED;
    if (!c || !a->codes || !a->scales || !b->codes || !b->scales) return MX_ERR_ARG;
    if ((fa->macro_cols && !a->macro_scales) || (fb->macro_cols && !b->macro_scales)) return MX_ERR_ARG;
    if ((fa->scale == MX_SCALE_NVFP4 && !a->tensor_scale) || (fb->scale == MX_SCALE_NVFP4 && !b->tensor_scale))
        return MX_ERR_ARG;
    if (!aligned16(c) || !aligned16(a->codes) || !aligned16(b->codes) || !aligned16(a->scales) ||
        !aligned16(b->scales))
        return MX_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int cb = c_dtype == MX_DTYPE_BF16;
    const uint8_t *ac = static_cast<const uint8_t*>(a->codes), *as = static_cast<const uint8_t*>(a->scales);
    const uint8_t *bc = static_cast<const uint8_t*>(b->codes), *bs = static_cast<const uint8_t*>(b->scales);
    if (!native)
        return hip_status(mxk::launch_gemm_upcvt(
            fa->scale, fa->block_cols, ac, as, fa->scale == MX_SCALE_NVFP4 ? a->tensor_scale : nullptr, fb->scale,
            fb->block_cols, bc, bs, fb->scale == MX_SCALE_NVFP4 ? b->tensor_scale : nullptr, c, M, N, K, ldc, cb, s,
            fa->macro_cols ? static_cast<const uint8_t*>(a->macro_scales) : nullptr,
            fb->macro_cols ? static_cast<const uint8_t*>(b->macro_scales) : nullptr));
    return hip_status(mxk::launch_gemm(fa->elem, ac, as, fb->elem, bc, bs, c, M, N, K, ldc, cb, s,
                                       fa->macro_cols ? static_cast<const uint8_t*>(a->macro_scales) : nullptr,
                                       fb->macro_cols ? static_cast<const uint8_t*>(b->macro_scales) : nullptr));
}

}  // extern "C"
