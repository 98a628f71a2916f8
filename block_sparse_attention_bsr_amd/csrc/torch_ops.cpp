// PyTorch operator registration of block-sparse attention over the C ABI.
//
// Two operators in the `bsr_attn` namespace, each a thin marshalling layer
// over the library's entry points (operand checks, output and workspace
// allocation through the caching allocator, the current stream, the C call):
//
//   attention_fwd(q, k, v, structure_id, scale, backward_schedule)
//       -> (O, row_max, row_denom)                              bsr_attn_fwd
//   attention_bwd(q, k, v, o, d_o, row_max, row_denom, structure_id, scale,
//                 backward_schedule) -> (dQ, dK, dV)
//                                          bsr_attn_bwd or bsr_attn_bwd_ds
//
// The forward operator's autograd kernel is registered on the operator itself
// (page "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: autograd on the native
// path is attached to the ops): it saves (Q, K, V, O, row_max, row_denom) and
// its backward calls attention_bwd with those statistics instead of
// recomputing them (page "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.1). The
// statistics are non-differentiable. attention_bwd's own autograd kernel
// refuses a second backward rather than return wrong second-order gradients.
//
// Both operators run here, in C++, so that an autograd step spends no time
// in Python beyond the call of attention_fwd itself. Their shape functions
// for fake and meta tensors are registered from Python.
//
// Operators cannot take a host object, so a structure is named by an integer
// id. The Python Structure registers its handle and each device plan it
// binds under that id (bsr_attn_torch_register*), and removes them before it
// destroys the handle; an operator holds the registry lock while it enqueues,
// so a structure cannot be destroyed under a running call.
#include <ATen/ATen.h>
#include <ATen/core/dispatch/Dispatcher.h>
#include <c10/core/DeviceGuard.h>
#include <c10/hip/HIPStream.h>
#include <torch/csrc/autograd/custom_function.h>
#include <torch/library.h>

#include <cstdint>
#include <limits>
#include <mutex>
#include <string>
#include <string_view>
#include <tuple>
#include <unordered_map>

#include "bsr_attn.h"

namespace {

using at::Tensor;
using Triple = std::tuple<Tensor, Tensor, Tensor>;

struct Registered {
    const bsr_attn_structure *s = nullptr;
    std::unordered_map<int, const void *> plans;  // device index -> bound device plan
};

std::mutex g_mu;
std::unordered_map<int64_t, Registered> g_structures;

int32_t dtype_code(at::ScalarType t) {
    switch (t) {
    case at::kFloat: return BSR_ATTN_F32;
    case at::kBFloat16: return BSR_ATTN_BF16;
    case at::kHalf: return BSR_ATTN_F16;
    default: TORCH_CHECK_TYPE(false, "unsupported dtype ", t, " (float32, bfloat16 or float16)");
    }
}

// q, k, v (and o, d_o): one GPU, one dtype, one [B, H, S, D] shape, contiguous.
void check_operands(const Tensor &q, std::initializer_list<std::pair<const char *, const Tensor *>> more) {
    TORCH_CHECK_VALUE(q.is_cuda(), "operands must be on a GPU device");
    TORCH_CHECK_VALUE(q.dim() == 4, "operands must be [batch, heads, seq_len, head_dim]");
    for (int64_t n : q.sizes())
        TORCH_CHECK_VALUE(n <= std::numeric_limits<int32_t>::max(), "operand dimension too large");
    TORCH_CHECK_VALUE(q.is_contiguous(), "q must be contiguous");
    for (const auto &[name, t] : more) {
        TORCH_CHECK_VALUE(t->device() == q.device() && t->scalar_type() == q.scalar_type() &&
                              t->sizes() == q.sizes(),
                          name, " must match q in device, dtype and shape");
        TORCH_CHECK_VALUE(t->is_contiguous(), name, " must be contiguous");
    }
}

void check_stats(const Tensor &q, const char *name, const Tensor &t) {
    TORCH_CHECK_VALUE(t.scalar_type() == at::kFloat && t.dim() == 3 && t.sizes() == q.sizes().slice(0, 3) &&
                          t.device() == q.device() && t.is_contiguous(),
                      name, " must be contiguous fp32 [B, H, S] on q's device");
}

bsr_attn_problem problem(const Tensor &q, double scale) {
    bsr_attn_problem p;
    p.batch = static_cast<int32_t>(q.size(0));
    p.heads = static_cast<int32_t>(q.size(1));
    p.seq_len = static_cast<int32_t>(q.size(2));
    p.head_dim = static_cast<int32_t>(q.size(3));
    p.dtype = dtype_code(q.scalar_type());
    p.scale = static_cast<float>(scale);
    return p;
}

void check_status(bsr_attn_status st, const char *entry) {
    TORCH_CHECK(st == BSR_ATTN_OK, entry, " failed (status ", static_cast<int>(st), "): ", bsr_attn_last_error());
}

// Runs f(structure, device plan) with the registry locked.
template <typename F> auto with_structure(int64_t id, int device, F &&f) {
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_structures.find(id);
    TORCH_CHECK_VALUE(it != g_structures.end(), "no live Structure with id ", id);
    auto plan = it->second.plans.find(device);
    TORCH_CHECK_VALUE(plan != it->second.plans.end(), "Structure ", id, " has no device plan bound on GPU ", device);
    return f(it->second.s, plan->second);
}

Tensor workspace(const bsr_attn_structure *s, const bsr_attn_problem &p, int backward, const Tensor &like,
                 size_t &nbytes) {
    nbytes = bsr_attn_workspace_bytes(s, &p, backward);
    return nbytes ? at::empty({static_cast<int64_t>(nbytes)}, like.options().dtype(at::kByte)) : Tensor();
}

void *ptr_or_null(const Tensor &t) { return t.defined() ? t.data_ptr() : nullptr; }

Triple attention_fwd_gpu(const Tensor &q, const Tensor &k, const Tensor &v, int64_t sid, double scale,
                         std::string_view) {
    check_operands(q, {{"k", &k}, {"v", &v}});
    const c10::DeviceGuard guard(q.device());
    const bsr_attn_problem p = problem(q, scale);
    Tensor o = at::empty_like(q);
    Tensor row_max = at::empty(q.sizes().slice(0, 3), q.options().dtype(at::kFloat));
    Tensor row_denom = at::empty_like(row_max);
    hipStream_t stream = c10::hip::getCurrentHIPStream(q.device().index()).stream();
    with_structure(sid, q.device().index(), [&](const bsr_attn_structure *s, const void *plan) {
        size_t nbytes = 0;
        Tensor ws = workspace(s, p, 0, q, nbytes);
        check_status(bsr_attn_fwd(s, plan, &p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  row_max.data_ptr<float>(), row_denom.data_ptr<float>(), ptr_or_null(ws), nbytes,
                                  stream),
                     "bsr_attn_fwd");
        return 0;
    });
    return {o, row_max, row_denom};
}

Triple attention_bwd_gpu(const Tensor &q, const Tensor &k, const Tensor &v, const Tensor &o, const Tensor &d_o,
                         const Tensor &row_max, const Tensor &row_denom, int64_t sid, double scale,
                         std::string_view schedule) {
    check_operands(q, {{"k", &k}, {"v", &v}, {"o", &o}, {"d_o", &d_o}});
    check_stats(q, "row_max", row_max);
    check_stats(q, "row_denom", row_denom);
    const bool store_ds = schedule == "store_ds";
    TORCH_CHECK_VALUE(store_ds || schedule == "recompute", "backward_schedule must be 'recompute' or 'store_ds'");
    const c10::DeviceGuard guard(q.device());
    const bsr_attn_problem p = problem(q, scale);
    Tensor dq = at::empty_like(q), dk = at::empty_like(q), dv = at::empty_like(q);
    hipStream_t stream = c10::hip::getCurrentHIPStream(q.device().index()).stream();
    with_structure(sid, q.device().index(), [&](const bsr_attn_structure *s, const void *plan) {
        size_t nbytes = 0;
        Tensor ws = workspace(s, p, store_ds ? 2 : 1, q, nbytes);
        auto entry = store_ds ? bsr_attn_bwd_ds : bsr_attn_bwd;
        check_status(entry(s, plan, &p, q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), d_o.data_ptr(),
                           row_max.data_ptr<float>(), row_denom.data_ptr<float>(), dq.data_ptr(), dk.data_ptr(),
                           dv.data_ptr(), ptr_or_null(ws), nbytes, stream),
                     store_ds ? "bsr_attn_bwd_ds" : "bsr_attn_bwd");
        return 0;
    });
    return {dq, dk, dv};
}

// Typed handles for calling the operators through the dispatcher (so that
// the backward reaches attention_bwd's own autograd kernel, and meta / fake
// tensors their shape functions).
const c10::TypedOperatorHandle<decltype(attention_fwd_gpu)> &fwd_op() {
    static const auto op = c10::Dispatcher::singleton()
                               .findSchemaOrThrow("bsr_attn::attention_fwd", "")
                               .typed<decltype(attention_fwd_gpu)>();
    return op;
}

const c10::TypedOperatorHandle<decltype(attention_bwd_gpu)> &bwd_op() {
    static const auto op = c10::Dispatcher::singleton()
                               .findSchemaOrThrow("bsr_attn::attention_bwd", "")
                               .typed<decltype(attention_bwd_gpu)>();
    return op;
}

using torch::autograd::AutogradContext;
using torch::autograd::variable_list;

struct AttentionFunction : public torch::autograd::Function<AttentionFunction> {
    static variable_list forward(AutogradContext *ctx, const Tensor &q, const Tensor &k, const Tensor &v,
                                 int64_t sid, double scale, const std::string &schedule) {
        Triple out;
        {
            at::AutoDispatchBelowADInplaceOrView below;
            out = fwd_op().call(q, k, v, sid, scale, schedule);
        }
        auto &[o, row_max, row_denom] = out;
        ctx->save_for_backward({q, k, v, o, row_max, row_denom});
        ctx->saved_data["sid"] = sid;
        ctx->saved_data["scale"] = scale;
        ctx->saved_data["schedule"] = schedule;
        ctx->mark_non_differentiable({row_max, row_denom});
        return {o, row_max, row_denom};
    }

    static variable_list backward(AutogradContext *ctx, variable_list grads) {
        const Tensor &d_o = grads[0];
        if (!d_o.defined()) return {Tensor(), Tensor(), Tensor(), Tensor(), Tensor(), Tensor()};
        const variable_list saved = ctx->get_saved_variables();
        const std::string schedule = ctx->saved_data["schedule"].toStringRef();
        auto [dq, dk, dv] = bwd_op().call(saved[0], saved[1], saved[2], saved[3], d_o.contiguous(), saved[4],
                                          saved[5], ctx->saved_data["sid"].toInt(),
                                          ctx->saved_data["scale"].toDouble(), schedule);
        return {dq, dk, dv, Tensor(), Tensor(), Tensor()};
    }
};

struct AttentionBackwardFunction : public torch::autograd::Function<AttentionBackwardFunction> {
    static variable_list forward(AutogradContext *, const Tensor &q, const Tensor &k, const Tensor &v,
                                 const Tensor &o, const Tensor &d_o, const Tensor &row_max, const Tensor &row_denom,
                                 int64_t sid, double scale, const std::string &schedule) {
        at::AutoDispatchBelowADInplaceOrView below;
        auto [dq, dk, dv] = bwd_op().call(q, k, v, o, d_o, row_max, row_denom, sid, scale, schedule);
        return {dq, dk, dv};
    }

    static variable_list backward(AutogradContext *, variable_list) {
        TORCH_CHECK(false, "bsr_attn::attention_bwd has no autograd formula: second-order gradients of "
                           "block-sparse attention are not supported");
    }
};

Triple attention_fwd_autograd(const Tensor &q, const Tensor &k, const Tensor &v, int64_t sid, double scale,
                              std::string_view schedule) {
    variable_list r = AttentionFunction::apply(q, k, v, sid, scale, std::string(schedule));
    return {r[0], r[1], r[2]};
}

Triple attention_bwd_autograd(const Tensor &q, const Tensor &k, const Tensor &v, const Tensor &o, const Tensor &d_o,
                              const Tensor &row_max, const Tensor &row_denom, int64_t sid, double scale,
                              std::string_view schedule) {
    variable_list r = AttentionBackwardFunction::apply(q, k, v, o, d_o, row_max, row_denom, sid, scale,
                                                       std::string(schedule));
    return {r[0], r[1], r[2]};
}

}  // namespace

TORCH_LIBRARY(bsr_attn, m) {
    m.set_python_module("block_sparse_attention_bsr_amd.autograd");
    m.def("attention_fwd(Tensor q, Tensor k, Tensor v, int structure_id, float scale, str backward_schedule) "
          "-> (Tensor, Tensor, Tensor)");
    m.def("attention_bwd(Tensor q, Tensor k, Tensor v, Tensor o, Tensor d_o, Tensor row_max, Tensor row_denom, "
          "int structure_id, float scale, str backward_schedule) -> (Tensor, Tensor, Tensor)");
}

TORCH_LIBRARY_IMPL(bsr_attn, CUDA, m) {
    m.impl("attention_fwd", &attention_fwd_gpu);
    m.impl("attention_bwd", &attention_bwd_gpu);
}

TORCH_LIBRARY_IMPL(bsr_attn, Autograd, m) {
    m.impl("attention_fwd", &attention_fwd_autograd);
    m.impl("attention_bwd", &attention_bwd_autograd);
}

// Registry of live structures, called from the Python Structure (ctypes).
// Return 0, or 1 for an invalid argument.
extern "C" {

__attribute__((visibility("default"))) int bsr_attn_torch_register(int64_t id, const bsr_attn_structure *s) {
    if (s == nullptr || id <= 0) return 1;
    std::lock_guard<std::mutex> lock(g_mu);
    g_structures[id].s = s;
    return 0;
}

__attribute__((visibility("default"))) int bsr_attn_torch_register_plan(int64_t id, int device, const void *plan) {
    if (plan == nullptr || device < 0) return 1;
    std::lock_guard<std::mutex> lock(g_mu);
    auto it = g_structures.find(id);
    if (it == g_structures.end()) return 1;
    it->second.plans[device] = plan;
    return 0;
}

__attribute__((visibility("default"))) void bsr_attn_torch_unregister(int64_t id) {
    std::lock_guard<std::mutex> lock(g_mu);
    g_structures.erase(id);
}

}  // extern "C"
