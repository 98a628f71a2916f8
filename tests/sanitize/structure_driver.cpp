// Host-side driver for the structure builder under AddressSanitizer and
// UndefinedBehaviorSanitizer (CPU only; built by tests/test_sanitizers.py
// with g++). It builds structures for many masks, valid and malformed, and
// walks every host entry point of csrc/structure.cpp: build, info, plan
// size and pack, plan binding, workspace sizes, destroy. Any invalid memory
// access or undefined behaviour aborts the run with a sanitizer report.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "internal.h"

namespace bsr {
// The library defines this in its C ABI file, which also dispatches to the
// HIP launchers; the driver only needs the message store.
static std::string g_msg;
void set_error(const std::string &msg) { g_msg = msg; }
}  // namespace bsr

static int failures = 0;
#define CHECK(c)                                                              \
    do {                                                                      \
        if (!(c)) {                                                           \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
            ++failures;                                                       \
        }                                                                     \
    } while (0)

// Exercise every host entry point on one structure.
static void walk(bsr_attn_structure *s) {
    bsr_attn_structure_info info{};
    CHECK(bsr_attn_structure_get_info(s, &info) == BSR_ATTN_OK);
    const size_t nbytes = bsr_attn_structure_plan_bytes(s);
    std::vector<int32_t> plan(nbytes / 4);
    CHECK(bsr_attn_structure_pack(s, plan.data(), nbytes) == BSR_ATTN_OK);
    CHECK(bsr_attn_structure_pack(s, plan.data(), nbytes - 4) == BSR_ATTN_ERR_INVALID_ARGUMENT);
    CHECK(plan[0] == 0x42535241);
    // plan offsets stay inside the packed array
    for (int h = 10; h <= 21; ++h) CHECK(plan[h] >= 0 && static_cast<size_t>(plan[h]) <= plan.size());
    // binding bookkeeping (fake, aligned device addresses; never dereferenced)
    const void *a = reinterpret_cast<const void *>(uintptr_t{1} << 20);
    const void *b = reinterpret_cast<const void *>((uintptr_t{1} << 20) + 4096);
    CHECK(bsr_attn_structure_bind_plan(s, a, nbytes) == BSR_ATTN_OK);
    CHECK(bsr_attn_structure_bind_plan(s, b, nbytes + 4) == BSR_ATTN_ERR_INVALID_ARGUMENT);
    CHECK(bsr::plan_is_bound(*s, a) && !bsr::plan_is_bound(*s, b));
    CHECK(bsr_attn_structure_unbind_plan(s, a) == BSR_ATTN_OK);
    CHECK(bsr_attn_structure_unbind_plan(s, a) == BSR_ATTN_ERR_INVALID_ARGUMENT);
    // workspace sizes for several problems (the launch structure they pick included)
    for (int64_t BH : {1, 2, 16, 64})
        for (int D : {16, 32, 64, 96, 128, 256, 400, 512})
            for (int dt : {0, 1, 2})
                for (int kind : {0, 1, 2}) {
                    const size_t w = bsr::call_workspace(bsr::launch_structure(*s, BH), BH,
                                                         int64_t{s->nb} * 128, D, dt, kind);
                    (void)w;
                }
    (void)bsr::spmm_workspace(*s, 512);
}

static void build_and_walk(int32_t nb, const std::vector<int32_t> &rp, const std::vector<int32_t> &ci,
                           int32_t split, bool expect_ok) {
    bsr_attn_structure *s = nullptr;
    const bsr_attn_status st =
        bsr_attn_build_structure(nb, rp.data(), ci.empty() ? nullptr : ci.data(), 128, split, &s);
    CHECK((st == BSR_ATTN_OK) == expect_ok);
    if (st == BSR_ATTN_OK) {
        walk(s);
        bsr_attn_destroy_structure(s);
    } else {
        CHECK(s == nullptr);
    }
}

static void from_mask(const std::vector<uint8_t> &m, int32_t nb, int32_t split) {
    std::vector<int32_t> rp(nb + 1, 0), ci;
    for (int32_t i = 0; i < nb; ++i) {
        for (int32_t j = 0; j < nb; ++j)
            if (m[static_cast<size_t>(i) * nb + j]) ci.push_back(j);
        rp[i + 1] = static_cast<int32_t>(ci.size());
    }
    build_and_walk(nb, rp, ci, split, true);
}

int main() {
    std::mt19937 rng(1234);
    // random masks of many sizes and densities, automatic and explicit splits
    for (int32_t nb : {1, 2, 3, 5, 8, 17, 64, 130}) {
        for (double dens : {0.0, 0.05, 0.3, 1.0}) {
            std::vector<uint8_t> m(static_cast<size_t>(nb) * nb);
            std::uniform_real_distribution<double> u(0.0, 1.0);
            for (auto &x : m) x = u(rng) < dens;
            for (int32_t split : {0, 1, 2, 7}) from_mask(m, nb, split);
        }
        // global mask: band, first row and first column
        std::vector<uint8_t> g(static_cast<size_t>(nb) * nb);
        for (int32_t i = 0; i < nb; ++i)
            for (int32_t j = 0; j < nb; ++j) g[static_cast<size_t>(i) * nb + j] = (i - j <= 1 && j - i <= 1) || !i || !j;
        from_mask(g, nb, 0);
    }
    // malformed structures: every one is rejected, none is read out of bounds
    build_and_walk(2, {0, 1, 2}, {0, 2}, 0, false);        // column out of range
    build_and_walk(2, {0, 2, 2}, {1, 0}, 0, false);        // not ascending
    build_and_walk(2, {0, 2, 3}, {0, 0, 1}, 0, false);     // repeated column
    build_and_walk(3, {0, 2, 1, 3}, {0, 1, 2}, 0, false);  // row_ptr decreasing
    build_and_walk(2, {1, 2, 3}, {0, 1, 0}, 0, false);     // row_ptr[0] != 0
    build_and_walk(2, {0, 3, 3}, {0, 1, 1}, 0, false);     // more than nb blocks in a row
    build_and_walk(2, {0, 1, 2}, {0, 1}, -1, false);       // negative split
    build_and_walk(0, {0}, {}, 0, false);                  // no block rows
    {
        bsr_attn_structure *s = nullptr;
        CHECK(bsr_attn_build_structure(2, nullptr, nullptr, 128, 0, &s) == BSR_ATTN_ERR_INVALID_ARGUMENT);
        const int32_t rp[3] = {0, 1, 2};
        CHECK(bsr_attn_build_structure(2, rp, nullptr, 128, 0, &s) == BSR_ATTN_ERR_INVALID_ARGUMENT);
        CHECK(bsr_attn_build_structure(2, rp, rp, 64, 0, &s) == BSR_ATTN_ERR_UNSUPPORTED);
        CHECK(bsr_attn_structure_get_info(nullptr, nullptr) == BSR_ATTN_ERR_INVALID_ARGUMENT);
        CHECK(bsr_attn_structure_plan_bytes(nullptr) == 0);
        bsr_attn_destroy_structure(nullptr);
    }
    std::printf("structure driver: %d failures\n", failures);
    return failures ? 1 : 0;
}
