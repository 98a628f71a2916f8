// C ABI: argument validation and dispatch to the HIP launchers. Every check
// runs before anything is enqueued, so a call that fails has launched nothing.
#include <algorithm>
#include <cmath>
#include <string>

#include "internal.h"

namespace bsr {

static thread_local std::string g_last_error;

void set_error(const std::string &msg) { g_last_error = msg; }

// kind: 0 forward, 1 backward, 2 backward that stores dS. fixed_workspace:
// the workspace is the library's own device array (bsr_attn_bwd_noalloc),
// whose address is looked up only after these checks pass.
static bsr_attn_status check_common(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                                    size_t workspace_bytes, const void *workspace, int kind,
                                    bool fixed_workspace = false) {
    if (!s) { set_error("structure is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (!d_plan) { set_error("d_plan is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (!p) { set_error("problem is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (p->batch < 1 || p->heads < 1) {
        set_error("batch and heads must be >= 1");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (p->dtype != BSR_ATTN_F32 && p->dtype != BSR_ATTN_BF16 && p->dtype != BSR_ATTN_F16) {
        set_error("dtype must be BSR_ATTN_F32, BSR_ATTN_BF16 or BSR_ATTN_F16");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (static_cast<int64_t>(p->seq_len) != static_cast<int64_t>(s->nb) * kBlock) {
        set_error("seq_len (" + std::to_string(p->seq_len) + ") must equal 128 * n_block_rows (" +
                  std::to_string(static_cast<int64_t>(s->nb) * kBlock) + ")");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (p->head_dim < 1) { set_error("head_dim must be >= 1"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (!supported_head_dim(p->dtype, p->head_dim)) {
        set_error("head_dim " + std::to_string(p->head_dim) + " is not supported for this dtype "
                  "(a multiple of 16, at most 512 for bf16/fp16 and 128 for fp32)");
        return BSR_ATTN_ERR_UNSUPPORTED;
    }
    if (!(std::isfinite(p->scale) && p->scale > 0.f)) {
        set_error("scale must be finite and > 0");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    const int64_t bh = static_cast<int64_t>(p->batch) * p->heads;
    const bsr_attn_structure &ls = launch_structure(*s, bh);
    const int64_t grid = bh * static_cast<int64_t>(std::max(ls.row_items.size(), ls.col_items.size()));
    const int64_t width = padded_head_dim(p->dtype, p->head_dim);
    if (grid > 0x7fffffffLL || bh * p->seq_len * width > (1LL << 40)) {
        set_error("problem too large");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (kind == 2 && p->dtype == BSR_ATTN_F32) {
        set_error("the dS-storing backward takes bf16 or fp16 operands");
        return BSR_ATTN_ERR_UNSUPPORTED;
    }
    if (!plan_is_bound(*s, d_plan)) {
        set_error("d_plan is not a device copy bound to this structure (bsr_attn_structure_bind_plan)");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    const size_t need = call_workspace(ls, bh, p->seq_len, p->head_dim, p->dtype, kind);
    if (workspace_bytes < need) {
        set_error("workspace too small: need " + std::to_string(need) + " bytes, got " +
                  std::to_string(workspace_bytes));
        return BSR_ATTN_ERR_WORKSPACE_TOO_SMALL;
    }
    if (need > 0 && !workspace && !fixed_workspace) {
        set_error("workspace is NULL");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    return BSR_ATTN_OK;
}

static bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// The launch runs on the structure's finer split when batch * heads is small
// (launch_structure), with that split's plan, embedded in the device plan.
static LaunchCommon launch_common(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                                  void *stream) {
    const int64_t bh = static_cast<int64_t>(p->batch) * p->heads;
    return LaunchCommon{&launch_structure(*s, bh),
                        static_cast<const int32_t *>(d_plan) + launch_plan_offset(*s, bh),
                        p->batch * p->heads, p->seq_len, p->head_dim, p->dtype, p->scale, stream};
}

}  // namespace bsr

extern "C" {

const char *bsr_attn_last_error(void) { return bsr::g_last_error.c_str(); }

size_t bsr_attn_workspace_bytes(const bsr_attn_structure *s, const bsr_attn_problem *p, int backward) {
    if (!s || !p || p->batch < 1 || p->heads < 1 || p->head_dim < 1 || backward < 0 || backward > 2 ||
        (backward == 2 && p->dtype == BSR_ATTN_F32) ||
        static_cast<int64_t>(p->seq_len) != static_cast<int64_t>(s->nb) * bsr::kBlock)
        return 0;
    const int64_t bh = static_cast<int64_t>(p->batch) * p->heads;
    return bsr::call_workspace(bsr::launch_structure(*s, bh), bh, p->seq_len, p->head_dim, p->dtype, backward);
}

namespace {
using FwdLauncher = int (*)(const bsr::LaunchCommon &, const void *, const void *, const void *, void *, float *,
                            float *, void *);

bsr_attn_status forward(FwdLauncher launch, const bsr_attn_structure *s, const void *d_plan,
                        const bsr_attn_problem *p, const void *q, const void *k, const void *v, void *o,
                        float *row_max, float *row_denom, void *workspace, size_t workspace_bytes, void *stream) {
    bsr_attn_status st = bsr::check_common(s, d_plan, p, workspace_bytes, workspace, 0);
    if (st != BSR_ATTN_OK) return st;
    const void *ptrs[] = {q, k, v, o, row_max, row_denom};
    const char *names[] = {"q", "k", "v", "o", "row_max", "row_denom"};
    for (int i = 0; i < 6; ++i) {
        if (!ptrs[i]) { bsr::set_error(std::string(names[i]) + " is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
        if (!bsr::aligned16(ptrs[i])) {
            bsr::set_error(std::string(names[i]) + " must be 16-byte aligned");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
    }
    const bsr::LaunchCommon c = bsr::launch_common(s, d_plan, p, stream);
    const int err = launch(c, q, k, v, o, row_max, row_denom, workspace);
    if (err != 0) {
        bsr::set_error(std::string("HIP launch failed: ") + bsr::hip_error_string(err));
        return BSR_ATTN_ERR_HIP;
    }
    bsr::set_error("");
    return BSR_ATTN_OK;
}
}  // namespace

bsr_attn_status bsr_attn_fwd(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                             const void *q, const void *k, const void *v, void *o, float *row_max,
                             float *row_denom, void *workspace, size_t workspace_bytes, void *stream) {
    return forward(bsr::launch_fwd, s, d_plan, p, q, k, v, o, row_max, row_denom, workspace, workspace_bytes,
                   stream);
}

bsr_attn_status bsr_attn_fwd_two_pass(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                                      const void *q, const void *k, const void *v, void *o, float *row_max,
                                      float *row_denom, void *workspace, size_t workspace_bytes, void *stream) {
    return forward(bsr::launch_fwd_two_pass, s, d_plan, p, q, k, v, o, row_max, row_denom, workspace,
                   workspace_bytes, stream);
}

namespace {
bsr_attn_status check_backward_pointers(const void *q, const void *k, const void *v, const void *o,
                                        const void *d_o, const float *row_max, const float *row_denom,
                                        const void *dq, const void *dk, const void *dv) {
    const void *ptrs[] = {q, k, v, o, d_o, row_max, row_denom, dq, dk, dv};
    const char *names[] = {"q", "k", "v", "o", "d_o", "row_max", "row_denom", "dq", "dk", "dv"};
    for (int i = 0; i < 10; ++i) {
        if (!ptrs[i]) { bsr::set_error(std::string(names[i]) + " is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
        if (!bsr::aligned16(ptrs[i])) {
            bsr::set_error(std::string(names[i]) + " must be 16-byte aligned");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
    }
    return BSR_ATTN_OK;
}

using BwdLauncher = int (*)(const bsr::LaunchCommon &, const void *, const void *, const void *, const void *,
                            const void *, const float *, const float *, void *, void *, void *, void *);

bsr_attn_status backward(BwdLauncher launch, int kind, const bsr_attn_structure *s, const void *d_plan,
                         const bsr_attn_problem *p, const void *q, const void *k, const void *v, const void *o,
                         const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                         void *workspace, size_t workspace_bytes, void *stream) {
    bsr_attn_status st = bsr::check_common(s, d_plan, p, workspace_bytes, workspace, kind);
    if (st != BSR_ATTN_OK) return st;
    st = check_backward_pointers(q, k, v, o, d_o, row_max, row_denom, dq, dk, dv);
    if (st != BSR_ATTN_OK) return st;
    const bsr::LaunchCommon c = bsr::launch_common(s, d_plan, p, stream);
    const int err = launch(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, workspace);
    if (err != 0) {
        bsr::set_error(std::string("HIP launch failed: ") + bsr::hip_error_string(err));
        return BSR_ATTN_ERR_HIP;
    }
    bsr::set_error("");
    return BSR_ATTN_OK;
}
}  // namespace

bsr_attn_status bsr_attn_bwd(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                             const void *q, const void *k, const void *v, const void *o, const void *d_o,
                             const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                             void *workspace, size_t workspace_bytes, void *stream) {
    return backward(bsr::launch_bwd, 1, s, d_plan, p, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, workspace,
                    workspace_bytes, stream);
}

bsr_attn_status bsr_attn_bwd_noalloc(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                                     const void *q, const void *k, const void *v, const void *o, const void *d_o,
                                     const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                                     void *stream) {
    if (s && p && p->batch >= 1 && p->heads >= 1 &&
        static_cast<int64_t>(p->seq_len) == static_cast<int64_t>(s->nb) * bsr::kBlock &&
        bsr::supported_head_dim(p->dtype, p->head_dim)) {
        const int64_t bh = static_cast<int64_t>(p->batch) * p->heads;
        const size_t need = bsr::call_workspace(bsr::launch_structure(*s, bh), bh, p->seq_len, p->head_dim,
                                                p->dtype, 1);
        if (need > bsr::kScratchBytes) {
            bsr::set_error("bsr_attn_bwd_noalloc: this problem needs " + std::to_string(need) +
                           " bytes of workspace, more than its fixed " + std::to_string(bsr::kScratchBytes) +
                           " (use bsr_attn_bwd with a caller workspace)");
            return BSR_ATTN_ERR_WORKSPACE_TOO_SMALL;
        }
    }
    // The other checks are bsr_attn_bwd's; the device array's address is
    // looked up only once they pass.
    bsr_attn_status st = bsr::check_common(s, d_plan, p, bsr::kScratchBytes, nullptr, 1, true);
    if (st != BSR_ATTN_OK) return st;
    st = check_backward_pointers(q, k, v, o, d_o, row_max, row_denom, dq, dk, dv);
    if (st != BSR_ATTN_OK) return st;
    void *ws = nullptr;
    const int err = bsr::scratch_pointer(&ws);
    if (err != 0) {
        bsr::set_error(std::string("device scratch lookup failed: ") + bsr::hip_error_string(err));
        return BSR_ATTN_ERR_HIP;
    }
    return backward(bsr::launch_bwd, 1, s, d_plan, p, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws,
                    bsr::kScratchBytes, stream);
}

bsr_attn_status bsr_attn_bwd_ds(const bsr_attn_structure *s, const void *d_plan, const bsr_attn_problem *p,
                                const void *q, const void *k, const void *v, const void *o, const void *d_o,
                                const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                                void *workspace, size_t workspace_bytes, void *stream) {
    return backward(bsr::launch_bwd_ds, 2, s, d_plan, p, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, workspace,
                    workspace_bytes, stream);
}

bsr_attn_status bsr_attn_mfma_probe(int32_t dtype, int32_t iters, float *sink, void *stream, double *flops) {
    if (dtype != BSR_ATTN_F32 && dtype != BSR_ATTN_BF16 && dtype != BSR_ATTN_F16) {
        bsr::set_error("dtype must be BSR_ATTN_F32, BSR_ATTN_BF16 or BSR_ATTN_F16");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (iters < 1 || !sink || !flops) {
        bsr::set_error("iters must be >= 1 and sink, flops non-NULL");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    const int err = bsr::launch_mfma_probe(dtype, iters, sink, stream, flops);
    if (err != 0) {
        bsr::set_error(std::string("HIP launch failed: ") + bsr::hip_error_string(err));
        return BSR_ATTN_ERR_HIP;
    }
    bsr::set_error("");
    return BSR_ATTN_OK;
}

size_t bsr_spmm_workspace_bytes(const bsr_attn_structure *s, int32_t n_cols) {
    if (!s || n_cols <= 0) return 0;
    return bsr::spmm_workspace(*s, n_cols);
}

bsr_attn_status bsr_spmm(const bsr_attn_structure *s, const void *d_plan, int32_t dtype, int32_t n_cols,
                         const void *blocks, const void *b, void *c, void *workspace, size_t workspace_bytes,
                         void *stream) {
    if (!s) { bsr::set_error("structure is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (!d_plan) { bsr::set_error("d_plan is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (!bsr::plan_is_bound(*s, d_plan)) {
        bsr::set_error("d_plan is not a device copy bound to this structure (bsr_attn_structure_bind_plan)");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (dtype != BSR_ATTN_F32 && dtype != BSR_ATTN_BF16 && dtype != BSR_ATTN_F16) {
        bsr::set_error("dtype must be BSR_ATTN_F32, BSR_ATTN_BF16 or BSR_ATTN_F16");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (n_cols <= 0) { bsr::set_error("n_cols must be positive"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (n_cols % 128 != 0) {
        bsr::set_error("n_cols must be a multiple of 128");
        return BSR_ATTN_ERR_UNSUPPORTED;
    }
    if (static_cast<int64_t>(s->nb) * bsr::kBlock * n_cols > (int64_t{1} << 40)) {
        bsr::set_error("problem too large");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    const void *ptrs[] = {blocks, b, c};
    const char *names[] = {"blocks", "b", "c"};
    for (int i = 0; i < 3; ++i) {
        if (!ptrs[i] && !(i == 0 && s->nnzb == 0)) {
            bsr::set_error(std::string(names[i]) + " is NULL");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
        if (ptrs[i] && !bsr::aligned16(ptrs[i])) {
            bsr::set_error(std::string(names[i]) + " must be 16-byte aligned");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
    }
    const size_t need = bsr::spmm_workspace(*s, n_cols);
    if (workspace_bytes < need || (need > 0 && !workspace)) {
        bsr::set_error("workspace too small: need " + std::to_string(need) + " bytes");
        return BSR_ATTN_ERR_WORKSPACE_TOO_SMALL;
    }
    bsr::SpmmCommon cm{s, static_cast<const int32_t *>(d_plan), n_cols, dtype, stream};
    const int err = bsr::launch_spmm(cm, blocks, b, c, workspace);
    if (err != 0) {
        bsr::set_error(std::string("HIP launch failed: ") + bsr::hip_error_string(err));
        return BSR_ATTN_ERR_HIP;
    }
    bsr::set_error("");
    return BSR_ATTN_OK;
}

}  // extern "C"
