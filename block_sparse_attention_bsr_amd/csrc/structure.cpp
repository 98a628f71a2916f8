// Host-side structure builder: validates a BSR block structure, builds its
// BSC transpose, splits long block rows / columns into segments, orders the
// work items longest first and packs the int32 plan the kernels read.
// No HIP calls: everything here runs (and is tested) on the CPU.
//
// Sources: the BSR encoding of a boolean block mask and the 128-block size
// (page "trnsparse 0.7.0 -> 0.9.0", benchmarks/bench_native_trn2.py); the
// host-built column-first (BSC) view used by the dK/dV pass (page
// "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.5.1); the split of output tiles
// balanced by stored blocks with one writer per tile (page
// "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.9.0), here at workgroup granularity
// with fp32 partials merged by a second kernel.
#include <algorithm>
#include <cstring>
#include <new>
#include <queue>
#include <utility>

#include "internal.h"

namespace {

using Item = std::array<int32_t, 4>;

// Split one line (row or column) of n blocks starting at `first` into
// segments of at most T blocks, as equal as possible, appending items and,
// when split, one merge entry.
void add_line(int32_t line, int32_t first, int32_t n, int32_t T, int32_t &slots,
              std::vector<Item> &items, std::vector<Item> &merges) {
    if (n <= T) {
        items.push_back({line, first, first + n, -1});
        return;
    }
    const int32_t nseg = (n + T - 1) / T;
    const int32_t slot0 = slots;
    int32_t pos = first;
    for (int32_t sgi = 0; sgi < nseg; ++sgi) {
        const int32_t len = n / nseg + (sgi < n % nseg ? 1 : 0);
        items.push_back({line, pos, pos + len, slot0 + sgi});
        pos += len;
    }
    merges.push_back({line, slot0, nseg, 0});
    slots += nseg;
}

// Longest first; ties by line then segment start, so the order is a pure
// function of the structure.
void order_items(std::vector<Item> &items) {
    std::stable_sort(items.begin(), items.end(), [](const Item &a, const Item &b) {
        const int32_t la = a[2] - a[1], lb = b[2] - b[1];
        if (la != lb) return la > lb;
        if (a[0] != b[0]) return a[0] < b[0];
        return a[1] < b[1];
    });
}

// Longest-processing-time-first assignment of the (already length-ordered)
// items of one head to `nq` work queues: each item goes to the queue with the
// least work so far (lowest index on ties). Output: nq + 1 offsets, then the
// item indices queue by queue, each queue in processing order.
std::vector<int32_t> queue_schedule(const std::vector<Item> &items, int32_t nq) {
    const int32_t n = static_cast<int32_t>(items.size());
    std::vector<std::vector<int32_t>> q(nq);
    using Load = std::pair<int64_t, int32_t>;  // (work, queue)
    std::priority_queue<Load, std::vector<Load>, std::greater<Load>> heap;
    for (int32_t j = 0; j < nq; ++j) heap.push({0, j});
    for (int32_t i = 0; i < n; ++i) {
        Load top = heap.top();
        heap.pop();
        q[top.second].push_back(i);
        // an empty line still costs its prologue and its stores
        top.first += std::max<int32_t>(1, items[i][2] - items[i][1]);
        heap.push(top);
    }
    std::vector<int32_t> out(nq + 1 + n);
    int32_t pos = 0;
    for (int32_t j = 0; j < nq; ++j) {
        out[j] = pos;
        for (int32_t i : q[j]) out[nq + 1 + pos++] = i;
    }
    out[nq] = pos;
    return out;
}

}  // namespace

namespace bsr {

// BSC transpose, split, work items, queue schedules and the packed plan of
// a validated structure, at split threshold `split` (0 = automatic).
static void fill(bsr_attn_structure *s, int32_t nb, const int32_t *row_ptr, const int32_t *col_idx, int32_t nnzb,
          int32_t split) {
    s->nb = nb;
    s->nnzb = nnzb;
    s->row_ptr.assign(row_ptr, row_ptr + nb + 1);
    if (nnzb > 0) s->col_idx.assign(col_idx, col_idx + nnzb);

    // BSC transpose: counting sort by column; rows come out ascending.
    s->col_ptr.assign(nb + 1, 0);
    for (int32_t p = 0; p < nnzb; ++p) s->col_ptr[s->col_idx[p] + 1]++;
    for (int32_t c = 0; c < nb; ++c) s->col_ptr[c + 1] += s->col_ptr[c];
    s->row_idx.assign(nnzb, 0);
    s->bsc_block.assign(nnzb, 0);
    std::vector<int32_t> next(s->col_ptr.begin(), s->col_ptr.end() - 1);
    for (int32_t r = 0; r < nb; ++r)
        for (int32_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
            const int32_t q = next[s->col_idx[p]]++;
            s->row_idx[q] = r;
            s->bsc_block[q] = p;
        }

    for (int32_t r = 0; r < nb; ++r) s->max_row = std::max(s->max_row, row_ptr[r + 1] - row_ptr[r]);
    for (int32_t c = 0; c < nb; ++c) s->max_col = std::max(s->max_col, s->col_ptr[c + 1] - s->col_ptr[c]);

    // Automatic split: one and a half times the mean line length, at least
    // 4; but no split at all when the longest line exceeds that by at most
    // one block, since shortening the longest item by one block gains less
    // than the two merge launches a split brings (measured on the random
    // 1 % mask: 75 vs 78 us per bf16 step, 518 vs 542 us per fp32 step;
    // at 5 %, two blocks over, splitting stays faster: 113 vs 117 us).
    int32_t T = split;
    if (T == 0) {
        const int64_t mean_ceil = (static_cast<int64_t>(nnzb) + nb - 1) / nb;
        T = static_cast<int32_t>(std::max<int64_t>(4, (3 * mean_ceil + 1) / 2));
        const int32_t longest = std::max(s->max_row, s->max_col);
        if (longest <= T + 1) T = std::max(T, longest);
    }
    s->split = T;

    for (int32_t r = 0; r < nb; ++r)
        add_line(r, row_ptr[r], row_ptr[r + 1] - row_ptr[r], T, s->n_row_slots, s->row_items, s->row_merges);
    for (int32_t c = 0; c < nb; ++c)
        add_line(c, s->col_ptr[c], s->col_ptr[c + 1] - s->col_ptr[c], T, s->n_col_slots, s->col_items,
                 s->col_merges);
    order_items(s->row_items);
    order_items(s->col_items);

    // Pack.
    std::vector<int32_t> &pl = s->plan;
    pl.assign(kHeaderInts, 0);
    auto append = [&pl](const int32_t *src, size_t n) -> int32_t {
        const size_t off = pl.size();
        pl.insert(pl.end(), src, src + n);
        while (pl.size() % 4) pl.push_back(0);  // keep 16-byte alignment for int4 reads
        return static_cast<int32_t>(off);
    };
    auto append_items = [&](const std::vector<Item> &v) -> int32_t {
        return append(v.empty() ? nullptr : v.data()->data(), v.size() * 4);
    };
    pl[H_MAGIC] = kPlanMagic;
    pl[H_VERSION] = kPlanVersion;
    pl[H_NB] = nb;
    pl[H_NNZB] = nnzb;
    pl[H_N_ROW_ITEMS] = static_cast<int32_t>(s->row_items.size());
    pl[H_N_COL_ITEMS] = static_cast<int32_t>(s->col_items.size());
    pl[H_N_ROW_MERGES] = static_cast<int32_t>(s->row_merges.size());
    pl[H_N_COL_MERGES] = static_cast<int32_t>(s->col_merges.size());
    pl[H_N_ROW_SLOTS] = s->n_row_slots;
    pl[H_N_COL_SLOTS] = s->n_col_slots;
    const int32_t o1 = append(s->col_idx.data(), s->col_idx.size());
    const int32_t o2 = append(s->row_idx.data(), s->row_idx.size());
    const int32_t o3 = append_items(s->row_items);
    const int32_t o4 = append_items(s->col_items);
    const int32_t o5 = append_items(s->row_merges);
    const int32_t o6 = append_items(s->col_merges);
    const int32_t o7 = append(s->row_ptr.data(), s->row_ptr.size());
    const int32_t o8 = append(s->col_ptr.data(), s->col_ptr.size());
    auto append_schedules = [&](const std::vector<Item> &items) -> int32_t {
        const int32_t table = append(nullptr, 0);
        pl.resize(pl.size() + 8, 0);  // kQueueLevels offsets, padded to 16 bytes
        for (int lv = 0; lv < kQueueLevels; ++lv) {
            const std::vector<int32_t> sc = queue_schedule(items, 1 << lv);
            pl[table + lv] = append(sc.data(), sc.size());
        }
        return table;
    };
    const int32_t o9 = append_schedules(s->row_items);
    const int32_t o10 = append_schedules(s->col_items);
    const int32_t o11 = append(s->bsc_block.data(), s->bsc_block.size());
    pl[H_OFF_COL_IDX] = o1;
    pl[H_OFF_ROW_IDX] = o2;
    pl[H_OFF_ROW_ITEMS] = o3;
    pl[H_OFF_COL_ITEMS] = o4;
    pl[H_OFF_ROW_MERGES] = o5;
    pl[H_OFF_COL_MERGES] = o6;
    pl[H_OFF_ROW_PTR] = o7;
    pl[H_OFF_COL_PTR] = o8;
    pl[H_OFF_ROW_SCHED] = o9;
    pl[H_OFF_COL_SCHED] = o10;
    pl[H_OFF_BSC_BLOCK] = o11;
}


static bsr_attn_status build(int32_t nb, const int32_t *row_ptr, const int32_t *col_idx,
                             int32_t block_size, int32_t split, bsr_attn_structure **out) {
    if (!out) { set_error("out is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    *out = nullptr;
    if (block_size != kBlock) {
        set_error("block_size must be 128 (got " + std::to_string(block_size) + ")");
        return BSR_ATTN_ERR_UNSUPPORTED;
    }
    if (nb < 1) { set_error("n_block_rows must be >= 1"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (nb > 32768) {  // keeps nb * nb and the sequence length within int32
        set_error("n_block_rows must be <= 32768");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    if (!row_ptr) { set_error("row_ptr is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (split < 0) { set_error("split_threshold must be >= 0"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (row_ptr[0] != 0) { set_error("row_ptr[0] must be 0"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    for (int32_t r = 0; r < nb; ++r) {
        if (row_ptr[r + 1] < row_ptr[r]) {
            set_error("row_ptr must be non-decreasing (row " + std::to_string(r) + ")");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
        if (row_ptr[r + 1] - row_ptr[r] > nb) {
            set_error("block row " + std::to_string(r) + " has more than nb blocks");
            return BSR_ATTN_ERR_INVALID_ARGUMENT;
        }
    }
    const int32_t nnzb = row_ptr[nb];
    if (nnzb > 0 && !col_idx) { set_error("col_idx is NULL"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    for (int32_t r = 0; r < nb; ++r) {
        for (int32_t p = row_ptr[r]; p < row_ptr[r + 1]; ++p) {
            const int32_t c = col_idx[p];
            if (c < 0 || c >= nb) {
                set_error("col_idx[" + std::to_string(p) + "] = " + std::to_string(c) + " out of range");
                return BSR_ATTN_ERR_INVALID_ARGUMENT;
            }
            if (p > row_ptr[r] && c <= col_idx[p - 1]) {
                set_error("col_idx must be strictly ascending within block row " + std::to_string(r));
                return BSR_ATTN_ERR_INVALID_ARGUMENT;
            }
        }
    }

    bsr_attn_structure *s = new (std::nothrow) bsr_attn_structure();
    if (!s) { set_error("host allocation failed"); return BSR_ATTN_ERR_HOST_ALLOC; }
    try {
        fill(s, nb, row_ptr, col_idx, nnzb, split);
        // A finer split of the same structure for launches over few (batch,
        // head) pairs (see kFineLaunchLimit): about one stored block per item
        // for 256 items, when that is finer than the automatic threshold. An
        // explicit threshold is kept as given.
        const int32_t fine_T = std::max<int32_t>(1, (nnzb + 255) / 256);
        if (split == 0 && fine_T < s->split) {
            std::unique_ptr<bsr_attn_structure> f(new bsr_attn_structure());
            fill(f.get(), nb, row_ptr, col_idx, nnzb, fine_T);
            std::vector<int32_t> &pl = s->plan;
            s->fine_offset = static_cast<int32_t>(pl.size());  // a multiple of 4: 16-byte aligned
            pl.insert(pl.end(), f->plan.begin(), f->plan.end());
            pl[H_OFF_FINE_PLAN] = s->fine_offset;
            s->fine = std::move(f);
        }
    } catch (const std::bad_alloc &) {
        delete s;
        set_error("host allocation failed");
        return BSR_ATTN_ERR_HOST_ALLOC;
    }
    *out = s;
    return BSR_ATTN_OK;
}


FwdWorkspace fwd_workspace(const bsr_attn_structure &s, int64_t BH, int D) {
    FwdWorkspace w{};
    const size_t rows = static_cast<size_t>(s.n_row_slots) * BH * kBlock;
    w.part_o = 0;
    w.part_m2 = align256(rows * D * sizeof(float));
    w.part_l = w.part_m2 + align256(rows * sizeof(float));
    w.part_mx = w.part_l + align256(rows * sizeof(float));
    w.total = s.n_row_slots ? w.part_mx + align256(rows * sizeof(float)) : 0;
    return w;
}

PadWorkspace pad_workspace(size_t instance_total, int64_t BH, int64_t S, int D, int dtype, int n) {
    PadWorkspace w{align256(instance_total), 0, instance_total};
    const int Dp = padded_head_dim(dtype, D);
    if (Dp == 0 || Dp == D) return w;
    w.tensor = align256(static_cast<size_t>(BH) * static_cast<size_t>(S) * Dp * elem_bytes(dtype));
    w.total = w.base + static_cast<size_t>(n) * w.tensor;
    return w;
}

WideWorkspace wide_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D, size_t e) {
    WideWorkspace w{};
    const size_t blocks = static_cast<size_t>(BH) * s.nnzb * kBlock * kBlock;
    const size_t rows = static_cast<size_t>(BH) * S;
    size_t off = 0;
    auto take = [&off](size_t bytes) {
        const size_t at = off;
        off += align256(bytes);
        return at;
    };
    w.delta = take(rows * 4);
    w.lse2 = take(rows * 4);
    w.p = take(blocks * e);
    w.ds = take(blocks * e);
    w.part_rows = take(static_cast<size_t>(BH) * s.n_row_slots * kBlock * D * 4);
    w.part_cols = take(static_cast<size_t>(BH) * s.n_col_slots * kBlock * D * 4);
    w.total = off;
    return w;
}

size_t instance_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int width, int dtype, int kind) {
    if (kind == 0) return fwd_workspace(s, BH, width).total;
    if (width > 256) return wide_workspace(s, BH, S, width, elem_bytes(dtype)).total;
    const size_t bwd = bwd_workspace(s, BH, S, width).total;
    if (kind == 1) return bwd;
    const size_t ds = static_cast<size_t>(BH) * s.nnzb * kBlock * kBlock * elem_bytes(dtype);
    return ds ? ds_offset(bwd) + ds : bwd;
}

size_t call_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D, int dtype, int kind) {
    const int Dp = padded_head_dim(dtype, D);
    if (Dp == 0) return 0;
    const size_t inst = instance_workspace(s, BH, S, Dp, dtype, kind);
    return pad_workspace(inst, BH, S, D, dtype, kind ? kBwdPadTensors : kFwdPadTensors).total;
}

bool plan_is_bound(const bsr_attn_structure &s, const void *d_plan) {
    std::lock_guard<std::mutex> lock(s.bound_mu);
    for (const auto &b : s.bound)
        if (b.first == d_plan) return true;
    return false;
}

size_t spmm_workspace(const bsr_attn_structure &s, int n_cols) {
    return static_cast<size_t>(s.n_row_slots) * kBlock * static_cast<size_t>(n_cols) * sizeof(float);
}

BwdWorkspace bwd_workspace(const bsr_attn_structure &s, int64_t BH, int64_t S, int D) {
    BwdWorkspace w{};
    const size_t nrow = static_cast<size_t>(BH) * S;
    w.delta = 0;
    w.lse2 = align256(nrow * sizeof(float));
    w.part_dq = w.lse2 + align256(nrow * sizeof(float));
    const size_t qsz = static_cast<size_t>(s.n_row_slots) * BH * kBlock * D * sizeof(float);
    const size_t ksz = static_cast<size_t>(s.n_col_slots) * BH * kBlock * D * sizeof(float);
    w.part_dk = w.part_dq + align256(qsz);
    w.part_dv = w.part_dk + align256(ksz);
    w.total = w.part_dv + align256(ksz);
    return w;
}

}  // namespace bsr

extern "C" {

bsr_attn_status bsr_attn_build_structure(int32_t n_block_rows, const int32_t *row_ptr,
                                         const int32_t *col_idx, int32_t block_size,
                                         int32_t split_threshold, bsr_attn_structure **out) {
    return bsr::build(n_block_rows, row_ptr, col_idx, block_size, split_threshold, out);
}

void bsr_attn_destroy_structure(bsr_attn_structure *s) { delete s; }

bsr_attn_status bsr_attn_structure_get_info(const bsr_attn_structure *s, bsr_attn_structure_info *info) {
    if (!s || !info) { bsr::set_error("NULL argument"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    info->n_block_rows = s->nb;
    info->nnzb = s->nnzb;
    info->split_threshold = s->split;
    info->n_row_items = static_cast<int32_t>(s->row_items.size());
    info->n_col_items = static_cast<int32_t>(s->col_items.size());
    info->n_row_merges = static_cast<int32_t>(s->row_merges.size());
    info->n_col_merges = static_cast<int32_t>(s->col_merges.size());
    info->n_row_slots = s->n_row_slots;
    info->n_col_slots = s->n_col_slots;
    info->max_row_blocks = s->max_row;
    info->max_col_blocks = s->max_col;
    info->fine_split_threshold = s->fine ? s->fine->split : 0;
    info->fine_n_row_items = s->fine ? static_cast<int32_t>(s->fine->row_items.size()) : 0;
    return BSR_ATTN_OK;
}

bsr_attn_status bsr_attn_structure_bind_plan(bsr_attn_structure *s, const void *d_plan, size_t bytes) {
    if (!s || !d_plan) { bsr::set_error("NULL argument"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    if (reinterpret_cast<uintptr_t>(d_plan) & 15u) {
        bsr::set_error("d_plan must be 16-byte aligned");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    const size_t need = s->plan.size() * sizeof(int32_t);
    if (bytes != need) {
        bsr::set_error("d_plan size " + std::to_string(bytes) + " is not this structure's plan size " +
                       std::to_string(need));
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    std::lock_guard<std::mutex> lock(s->bound_mu);
    for (const auto &b : s->bound)
        if (b.first == d_plan) return BSR_ATTN_OK;
    if (s->bound.size() >= static_cast<size_t>(bsr::kMaxBoundPlans)) {
        bsr::set_error("too many device plans bound to this structure (at most " +
                       std::to_string(bsr::kMaxBoundPlans) + "); unbind one first");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    try {
        s->bound.emplace_back(d_plan, bytes);
    } catch (const std::bad_alloc &) {
        bsr::set_error("host allocation failed");
        return BSR_ATTN_ERR_HOST_ALLOC;
    }
    return BSR_ATTN_OK;
}

bsr_attn_status bsr_attn_structure_unbind_plan(bsr_attn_structure *s, const void *d_plan) {
    if (!s || !d_plan) { bsr::set_error("NULL argument"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    std::lock_guard<std::mutex> lock(s->bound_mu);
    for (size_t i = 0; i < s->bound.size(); ++i)
        if (s->bound[i].first == d_plan) {
            s->bound.erase(s->bound.begin() + static_cast<std::ptrdiff_t>(i));
            return BSR_ATTN_OK;
        }
    bsr::set_error("d_plan is not bound to this structure");
    return BSR_ATTN_ERR_INVALID_ARGUMENT;
}

size_t bsr_attn_structure_plan_bytes(const bsr_attn_structure *s) {
    return s ? s->plan.size() * sizeof(int32_t) : 0;
}

bsr_attn_status bsr_attn_structure_pack(const bsr_attn_structure *s, void *host_dst, size_t bytes) {
    if (!s || !host_dst) { bsr::set_error("NULL argument"); return BSR_ATTN_ERR_INVALID_ARGUMENT; }
    const size_t need = s->plan.size() * sizeof(int32_t);
    if (bytes < need) {
        bsr::set_error("plan buffer too small: need " + std::to_string(need) + " bytes");
        return BSR_ATTN_ERR_INVALID_ARGUMENT;
    }
    std::memcpy(host_dst, s->plan.data(), need);
    return BSR_ATTN_OK;
}

}  // extern "C"
