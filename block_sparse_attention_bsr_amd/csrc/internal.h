// Internal declarations shared by the host structure builder, the C ABI and
// the HIP launchers. Not part of the public interface.
#pragma once

#include <array>
#include <cstddef>
#include <cstdint>
#include <memory>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "bsr_attn.h"

struct bsr_attn_structure {
    int32_t nb = 0, nnzb = 0, split = 0;
    std::vector<int32_t> row_ptr, col_idx;  // BSR
    std::vector<int32_t> col_ptr, row_idx;  // BSC (block rows ascending per column)
    std::vector<int32_t> bsc_block;         // BSR position of each BSC entry
    // work items {line, first, end, slot}; merges {line, first slot, count, 0}
    std::vector<std::array<int32_t, 4>> row_items, col_items, row_merges, col_merges;
    int32_t n_row_slots = 0, n_col_slots = 0, max_row = 0, max_col = 0;
    std::vector<int32_t> plan;  // packed int32 plan (see bsr_attn.h)
    // The same structure split finer (automatic threshold only), for launches
    // with too few (batch, head) pairs to fill the chip; its packed plan is
    // embedded in `plan` at int32 offset fine_offset.
    std::unique_ptr<bsr_attn_structure> fine;
    int32_t fine_offset = 0;
    // Device copies of `plan` the caller has bound (pointer, bytes): fwd/bwd
    // accept only these as d_plan.
    mutable std::mutex bound_mu;
    std::vector<std::pair<const void *, size_t>> bound;
};

namespace bsr {

constexpr int32_t kBlock = 128;
constexpr int32_t kPlanMagic = 0x42535241;
constexpr int32_t kPlanVersion = 5;
constexpr int kHeaderInts = 24;

// header field indices
enum : int {
    H_MAGIC = 0, H_VERSION, H_NB, H_NNZB, H_N_ROW_ITEMS, H_N_COL_ITEMS, H_N_ROW_MERGES,
    H_N_COL_MERGES, H_N_ROW_SLOTS, H_N_COL_SLOTS, H_OFF_COL_IDX, H_OFF_ROW_IDX,
    H_OFF_ROW_ITEMS, H_OFF_COL_ITEMS, H_OFF_ROW_MERGES, H_OFF_COL_MERGES, H_OFF_ROW_PTR,
    H_OFF_COL_PTR, H_OFF_ROW_SCHED, H_OFF_COL_SCHED, H_OFF_BSC_BLOCK, H_OFF_FINE_PLAN
};

// A launch whose forward would have at most this many workgroups (batch *
// heads * row items; a quarter of MI355X's 256 compute units) runs on the
// structure's finer split, when it has one: few long items would otherwise
// leave most of the chip idle (one head of four block rows: four workgroups).
constexpr int64_t kFineLaunchLimit = 64;

// The structure a launch over BH (batch, head) pairs runs on, and the offset
// (int32) of its plan within the packed plan.
inline const bsr_attn_structure &launch_structure(const bsr_attn_structure &s, int64_t BH) {
    if (s.fine && BH * static_cast<int64_t>(s.row_items.size()) <= kFineLaunchLimit) return *s.fine;
    return s;
}
inline int32_t launch_plan_offset(const bsr_attn_structure &s, int64_t BH) {
    return &launch_structure(s, BH) == &s ? 0 : s.fine_offset;
}

// Per-head work queues: schedules for 1, 2, 4, ..., kMaxQueues queues.
constexpr int kQueueLevels = 7;
constexpr int kMaxQueues = 1 << (kQueueLevels - 1);

void set_error(const std::string &msg);

// Device plans a structure accepts (bsr_attn_structure_bind_plan).
constexpr int kMaxBoundPlans = 64;
bool plan_is_bound(const bsr_attn_structure &s, const void *d_plan);

// Workspace carve-up (byte offsets, each 256-aligned).
struct FwdWorkspace { size_t part_o, part_m2, part_l, part_mx, total; };
struct BwdWorkspace { size_t delta, lse2, part_dq, part_dk, part_dv, total; };
// Wide heads (head_dim 512), materialised blocks: S and dP fp32, P and dS in
// the operand dtype (e bytes), [BH][nnzb][128][128] each; SpMM partials per
// split row ([BH][row slots][128][D] fp32) and per split column (shared by
// dV, then dK). The forward uses s, p and part_rows.
// The head_dim 512 backward's workspace: row terms, P and dS blocks, fp32
// partials of split rows and columns.
struct WideWorkspace { size_t delta, lse2, p, ds, part_rows, part_cols, total; };
WideWorkspace wide_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D, size_t e);
FwdWorkspace fwd_workspace(const bsr_attn_structure &s, int64_t BH, int D);
BwdWorkspace bwd_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D);

// Launchers (kernels.hip). They assume validated arguments and return a HIP
// error code (0 = success) from the launch checks.
struct LaunchCommon {
    const bsr_attn_structure *s;
    const int32_t *d_plan;
    int BH, S, D, dtype;
    float scale;
    void *stream;
};

int launch_fwd(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o,
               float *row_max, float *row_denom, void *workspace);
int launch_fwd_two_pass(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o,
                        float *row_max, float *row_denom, void *workspace);
int launch_bwd_ds(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o,
                  const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                  void *ws);
int launch_bwd(const LaunchCommon &c, const void *q, const void *k, const void *v,
               const void *o, const void *d_o, const float *row_max, const float *row_denom,
               void *dq, void *dk, void *dv, void *workspace);
// Block-sparse times dense on the same plan.
struct SpmmCommon {
    const bsr_attn_structure *s;
    const int32_t *d_plan;
    int n_cols, dtype;
    void *stream;
};
int launch_spmm(const SpmmCommon &c, const void *blocks, const void *b, void *c_out, void *workspace);
// MFMA-loop probe (kernels.hip): enqueues the probe; *flops = its matrix work.
int launch_mfma_probe(int dtype, int iters, float *sink, void *stream, double *flops);
size_t spmm_workspace(const bsr_attn_structure &s, int n_cols);
const char *hip_error_string(int err);
// Size of the device array the no-allocation backward uses as its workspace,
// and its address on the current device (looked up on the first call on each
// device); returns a HIP error code.
constexpr size_t kScratchBytes = size_t{32} << 20;
int scratch_pointer(void **out);

// Records a timing event pair around one kernel launch on `stream` while
// bsr_attn_timing_begin() is active on this thread (timing.cpp); otherwise
// does nothing. The entry is named "<role><<dtype>,<head_dim>>" (",<head_dim>"
// omitted when head_dim is 0).
class KernelTimer {
  public:
    KernelTimer(const char *role, const char *dtype, int head_dim, void *stream);
    ~KernelTimer();
    KernelTimer(const KernelTimer &) = delete;
    KernelTimer &operator=(const KernelTimer &) = delete;

  private:
    void *stream_;
    void *stop_ = nullptr;
};
// Head dims with kernel instances of their own.
inline bool native_head_dim(int dtype, int D) {
    if (dtype == BSR_ATTN_BF16 || dtype == BSR_ATTN_F16) return D == 32 || D == 64 || D == 128 || D == 256 || D == 512;
    if (dtype == BSR_ATTN_F32) return D == 32 || D == 64 || D == 128;
    return false;
}
// The width a call runs at: its own head dim when that has an instance, else
// (for a multiple of 16) the next instantiated width, on zero-padded copies
// of the operands. 0 = not supported.
inline int padded_head_dim(int dtype, int D) {
    if (D < 16 || D % 16 != 0) return 0;
    for (int w = 32; w <= 512; w *= 2)
        if (D <= w && native_head_dim(dtype, w)) return w;
    return 0;
}
inline bool supported_head_dim(int dtype, int D) { return padded_head_dim(dtype, D) != 0; }
inline size_t elem_bytes(int dtype) { return dtype == BSR_ATTN_F32 ? 4 : 2; }

// Padded operand copies of a call whose head dim runs padded: `n` tensors of
// BH*S rows of the padded width, placed after the instance's own workspace.
// The forward pads Q, K, V and O (4), the backward Q, K, V, O, dO, dQ, dK, dV (8).
struct PadWorkspace { size_t base, tensor, total; };
PadWorkspace pad_workspace(size_t instance_total, int64_t BH, int64_t S, int D, int dtype, int n);
constexpr int kFwdPadTensors = 4, kBwdPadTensors = 8;
// Call kinds: 0 forward, 1 backward, 2 backward that stores dS.
// Workspace of the kernels of a call at head-dim width `width`, and the total
// of a call (with the padded operand copies when the head dim runs padded).
size_t instance_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int width, int dtype, int kind);
size_t call_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D, int dtype, int kind);
inline size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }
// The dS-storing backward keeps dS^T blocks ([BH][nnzb][128][128], operand
// dtype) after the backward's own carve-up.
inline size_t ds_offset(size_t bwd_total) { return align256(bwd_total); }

}  // namespace bsr
