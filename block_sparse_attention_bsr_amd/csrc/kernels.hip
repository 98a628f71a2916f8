// HIP kernels (CDNA4 / gfx950) for BSR block-sparse attention, and their
// launchers.
//
//   fwd_kernel        one workgroup per (row item, batch*head): the 128
//                     queries of a block row (or a segment of its stored
//                     blocks); online softmax over the stored key blocks;
//                     O = P V (also the two-pass form's statistics and output
//                     passes).
//   fwd_pair_kernel   the same at head_dim 256, two waves per SIMD split by
//                     role (scores and softmax / the accumulator).
//   fwd_merge_kernel  log-sum-exp merge of the fp32 partials of split rows.
//   dq_kernel         row-first dQ: one workgroup per (row item,
//                     batch*head); also forms delta = rowsum(dO * O) and the
//                     base-2 log-sum-exp of its rows, which the dK/dV pass
//                     reads. dq_pair_kernel: the same at head_dim 256, split
//                     by role.
//   dkdv_*            column-first dK/dV over the BSC view: dkdv_queue_kernel
//                     (16-bit, head_dim 32/64: per-head work queues),
//                     dkdv_pair_kernel (16-bit, 128: queues, two waves per
//                     SIMD split by role), dkdv_wide_pair_kernel (16-bit,
//                     256), dkdv_kernel (fp32); each optionally stores dS.
//   prep_kernel, dq_ds_kernel
//                     the dS-storing backward's row terms and its dQ = dS K.
//   sum_partials      fixed-order sum of split-line partials (dQ, dK, dV).
//   spmm_kernel, spmm_sum_kernel, sddmm_bwd_kernel
//                     block-sparse times dense on the same structure, and the
//                     head_dim 512 backward's P and dS blocks.
//   repack_kernel     zero-padded copies for head dims without an instance.
//   mfma_probe_kernel register-only product loop (the measured MFMA ceiling).
//
// Sources: page "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0 (forward in one
// launch with the statistics on chip; backward as dQ row-first plus dK/dV
// column-first) and 0.9.0 (bf16 operands, fp32 accumulation, fp32 statistics,
// output tiles balanced by stored blocks with one writer each); page
// "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.4.4 (stable softmax from row max
// and row sum, weights @ V accumulated across the key blocks of a row), 0.5.0
// (delta identity), 0.5.1 (the dQ / dK / dV accumulations and the BSC view),
// 0.6.0 (head_dim above 128 tiled along the contraction).
//
// Layout choices (MI355X-first, not taken from the pages):
//   * Every product runs on 32x32 MFMA tiles (bf16: v_mfma_f32_32x32x16_bf16,
//     fp32: v_mfma_f32_32x32x2_f32), fp32 accumulation.
//   * A workgroup is 4 waves (8 in the pair kernels, two per SIMD); each wave
//     (pair of waves) owns 32 rows (queries in fwd/dQ, keys in dK/dV) and
//     keeps its operand fragments in registers.
//   * Scores are produced so that a lane owns one output row's column of the
//     score tile (S^T = K Q^T in fwd/dQ; S = Q K^T in dK/dV). The MFMA result
//     layout then feeds the next product's B operand directly, and per-row
//     softmax statistics are per-lane scalars in fwd/dQ.
//   * Streamed tiles (K/V in fwd and dQ, Q/dO in dK/dV) are staged in LDS,
//     row-major with an XOR swizzle of 16-byte chunks; operands that contract
//     over the tile's rows are read with ds_read_b64_tr_b16 (bf16) straight
//     from the row-major tile, so no transposed copy is kept.
//   * exp is evaluated as exp2 with scale*log2(e) folded into the scores; the
//     statistics are returned in natural-log units.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <type_traits>
#include <vector>

#include "internal.h"

namespace bsr {
namespace {

template <typename T> constexpr const char *dtype_name() {
    return std::is_same<T, float>::value ? "fp32" : std::is_same<T, __bf16>::value ? "bf16" : "fp16";
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) short s16x8;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr int BLK = 128;
constexpr int NT = 256;  // threads per workgroup (4 waves)
constexpr float LOG2E = 1.4426950408889634f;

// ---------------------------------------------------------------------------
// Operand traits: the MFMA, its k-width and the result-row -> key map.
// For a 32x32 MFMA result, lane l holds column l%32 and rows
// r(v) = 8*(v/4) + 4*(l/32) + v%4 for its 16 values v. Loading the A operand
// of the score product with rows permuted by pi() makes the result values of
// a lane, taken in order, exactly the k-fragment the next MFMA's B operand
// expects (k = 8*(l/32) + e for bf16, k = l/32 for fp32, per k-step).
// ---------------------------------------------------------------------------
template <typename T> struct Op;

template <> struct Op<__bf16> {
    using frag = bf16x8;
    static constexpr int KW = 16;  // k per MFMA
    static constexpr int KL = 8;   // k per lane per MFMA
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int pi(int r) {  // swap bits 2 and 3
        return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
    }
    static __device__ __forceinline__ frag pack(const f32x16 &x, int v0) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = static_cast<__bf16>(x[v0 + e]);
        return f;
    }
};

template <> struct Op<_Float16> {
    using frag = f16x8;
    static constexpr int KW = 16;
    static constexpr int KL = 8;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int pi(int r) { return Op<__bf16>::pi(r); }
    static __device__ __forceinline__ frag pack(const f32x16 &x, int v0) {
        frag f;
#pragma unroll
        for (int e = 0; e < 8; ++e) f[e] = static_cast<_Float16>(x[v0 + e]);
        return f;
    }
};

template <> struct Op<float> {
    using frag = float;
    static constexpr int KW = 2;
    static constexpr int KL = 1;
    static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    static __device__ __forceinline__ int pi(int r) {  // 8a + 4h + b -> 8a + 2b + h
        return (r & ~7) | ((r & 3) << 1) | ((r >> 2) & 1);
    }
    static __device__ __forceinline__ frag pack(const f32x16 &x, int v0) { return x[v0]; }
};

// ---------------------------------------------------------------------------
// LDS tiles: `rows` x D, row-major.
//   bf16: 16-byte chunks, physical chunk = chunk ^ swz(row), swz in [0, 8).
//         Conflict-free for the two access patterns used: 8 lanes reading the
//         same chunk of rows {0,1,2,3,8,9,10,11}+x (pi-permuted row reads) and
//         16 lanes reading 2 chunks of 4 consecutive rows (transposing reads).
//   fp32 (TileF4, the double-buffered kernels): the same 16-byte chunk map.
//   fp32 (Tile<float>, the SpMM's synchronous staging): dword granularity,
//         physical column = col ^ (row & 31).
// ---------------------------------------------------------------------------
// Chunk swizzle of a row. Rows of 16+ chunks use a 4-bit XOR map, linear in
// the row bits (b0 -> 6, b1 -> 12, b2 -> 8, b3 -> 1); it keeps both access
// patterns conflict-free whether LDS serves 16-byte reads in 8-lane phases
// over 32 banks or in 16-lane phases over 64 banks. 8-chunk rows (D = 64)
// use a 3-bit map with the same property for 32 banks.
template <int CHUNKS> __device__ __forceinline__ int swz(int row) {
    if constexpr (CHUNKS >= 16) {
        return ((row & 1) ? 6 : 0) ^ ((row & 2) ? 12 : 0) ^ ((row & 4) ? 8 : 0) ^ ((row & 8) ? 1 : 0);
    } else if constexpr (CHUNKS == 8) {
        return ((row & 3) << 1) | ((row >> 3) & 1);
    } else {
        // 4-chunk rows (64 bytes, head_dim 32): four rows share a bank row, so
        // rows r, r + 4, r + 8, r + 12 get distinct chunk positions.
        static_assert(CHUNKS == 4, "chunks per row");
        return (row >> 2) & 3;
    }
}

template <typename T, int D> struct Tile;

// 16-bit element tiles (bf16 and fp16 share the layout and the reads).
template <typename H, int D> struct Tile16 {
    using frag = typename Op<H>::frag;
    static_assert(D == 32 || D % 64 == 0, "16-bit tiles: 4 chunks per row or a multiple of 8");
    static __device__ __forceinline__ uint32_t off(int row, int chunk) {
        return row * (D * 2) + ((chunk ^ swz<D / 8>(row)) << 4);
    }
    // A/B fragment along a row: 8 consecutive k (= columns k0..k0+7).
    static __device__ __forceinline__ frag frag_row(const char *lds, int row, int k0) {
        return *reinterpret_cast<const frag *>(lds + off(row, k0 >> 3));
    }
    // A/B fragment whose k runs down the tile's rows: lane gets rows
    // k0 + 8*(lane/32) + e (e = 0..7) of column c0 + lane%32.
    static __device__ __forceinline__ frag frag_tr(const char *lds, int k0, int c0, int lane) {
        const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
        const int chunk = col >> 3;
        const int sub = 8 * (lane & 1);
        const int r0 = k0 + 8 * (lane >> 5) + ((lane & 15) >> 2);
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(lds + off(r0, chunk) + sub));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4 *)(lds + off(r0 + 4, chunk) + sub));
        s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        return __builtin_bit_cast(frag, both);
    }
};
template <int D> struct Tile<__bf16, D> : Tile16<__bf16, D> {};
template <int D> struct Tile<_Float16, D> : Tile16<_Float16, D> {};

template <int D> struct Tile<float, D> {
    static_assert(D % 32 == 0, "fp32 tiles need at least 32 columns");
    static __device__ __forceinline__ uint32_t idx(int row, int col) {
        return row * D + (col ^ (row & 31));
    }
    // Stage rows [0, ROWS) of a global tile whose rows are `ld` floats apart.
    template <int ROWS>
    static __device__ __forceinline__ void stage_strided(char *lds, const float *g, size_t ld, int tid) {
        constexpr int CH = D / 4;
        constexpr int PER = ROWS * CH / NT;
        static_assert(ROWS * CH % NT == 0, "tile not divisible among threads");
        float4 tmp[PER];
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int id = i * NT + tid, row = id / CH, c = id % CH;
            tmp[i] = *reinterpret_cast<const float4 *>(g + row * ld + c * 4);
        }
        float *l = reinterpret_cast<float *>(lds);
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int id = i * NT + tid, row = id / CH, c = id % CH;
            l[idx(row, 4 * c)] = tmp[i].x;
            l[idx(row, 4 * c + 1)] = tmp[i].y;
            l[idx(row, 4 * c + 2)] = tmp[i].z;
            l[idx(row, 4 * c + 3)] = tmp[i].w;
        }
    }
    static __device__ __forceinline__ float frag_row(const char *lds, int row, int k0) {
        return reinterpret_cast<const float *>(lds)[idx(row, k0)];
    }
    static __device__ __forceinline__ float frag_tr(const char *lds, int k0, int c0, int lane) {
        return reinterpret_cast<const float *>(lds)[idx(k0 + (lane >> 5), c0 + (lane & 31))];
    }
};

// fp32 tiles staged by LDS-DMA: row-major, 16-byte chunks (four floats)
// XOR-swizzled per row with the 16-bit tiles' map (chunk ^ swz(row)), since
// the copies write whole 16-byte chunks. The fp32 products read one float per
// lane: the row reads of 32 rows then meet at most two to a bank, which their
// one read per 64-cycle product leaves far from the LDS limit.
template <int D> struct TileF4 {
    static_assert(D % 32 == 0, "fp32 tiles need at least 32 columns");
    static __device__ __forceinline__ uint32_t off(int row, int col) {
        return row * (D * 4) + (((col >> 2) ^ swz<D / 4>(row)) << 4) + 4 * (col & 3);
    }
    static __device__ __forceinline__ float frag_row(const char *lds, int row, int k0) {
        return *reinterpret_cast<const float *>(lds + off(row, k0));
    }
    static __device__ __forceinline__ float frag_tr(const char *lds, int k0, int c0, int lane) {
        return *reinterpret_cast<const float *>(lds + off(k0 + (lane >> 5), c0 + (lane & 31)));
    }
};
// The tile layout of the double-buffered (LDS-DMA) kernels.
template <typename T, int D>
using ATile = typename std::conditional<sizeof(T) == 2, Tile<T, D>, TileF4<D>>::type;

// ---------------------------------------------------------------------------
// Asynchronous staging: global_load_lds_dwordx4 writes each lane's 16
// bytes straight into LDS at (wave-uniform base + 16 * lane), so the swizzle
// is applied on the global side: the lane that owns physical chunk pc of a
// row fetches logical chunk pc ^ swz(row). Completion is tracked with
// explicit vmcnt waits; the kernels issue no other vector-memory loads while
// a stage is in flight.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// The LDS-DMA loads are issued through inline assembly so that the compiler
// does not track them: its own wait insertion would otherwise stall on every
// LDS read it cannot prove disjoint from a transfer in flight. Their
// completion is covered by the explicit vmcnt waits below; any vector-memory
// load the compiler issues itself can only make those waits stricter (loads
// complete in order). M0 holds the wave-uniform LDS destination; one wait
// state separates the M0 write from the load. The compiler reserves M0 and
// does not preserve it across the asm; that is safe here because nothing
// else in these kernels reads M0 (on gfx950 LDS instructions do not use it,
// and the kernels use no other M0 consumer: no movrel, message or GDS
// instructions, no compiler-issued LDS-DMA). The generated code has been
// checked for that: every M0 access is one of these sequences.
__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void *)p)));
}
// 16 bytes per lane, from a wave-uniform base address plus a per-lane 32-bit
// byte offset.
__device__ __forceinline__ void dma16_sbase(const void *base, uint32_t off, uint32_t m0) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "s"(m0)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma4(const void *g, const void *lds) {
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off" ::"v"(g), "s"(lds_addr(lds))
                 : "memory", "m0");
}

template <int RB, int ROWS, int NTH = NT>
struct AsyncRows {  // rows of RB bytes
    static constexpr int CH = RB / 16;
    static constexpr int LOADS = ROWS * CH / NTH;  // per thread
    static_assert(ROWS * CH % NTH == 0, "tile not divisible among threads");
    // Load i covers rows i*R .. i*R + R - 1. The swizzle depends on row % 16
    // only, so the per-lane source offsets repeat with period P loads and
    // just P of them are kept (in VGPRs); the others add a constant.
    static constexpr int R = NTH / CH;
    static constexpr int P = (R % 16 == 0 || LOADS == 1) ? 1 : (16 / R < LOADS ? 16 / R : LOADS);
    static_assert(R % 16 == 0 || 16 % R == 0, "swizzle period");
    // Per-lane source offsets (bytes, relative to the tile's first row) and
    // the wave's LDS offset: the same for every stage, computed once.
    struct Plan {
        uint32_t goff[P];
        uint32_t wave_lds;
    };
    static __device__ __forceinline__ Plan plan(int tid) {
        Plan pl;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = i * NTH + tid, row = p / CH, pc = p % CH;
            const int c = pc ^ swz<CH>(row);
            pl.goff[i] = static_cast<uint32_t>(row * RB + c * 16);
        }
        pl.wave_lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((tid & ~63) * 16));
        return pl;
    }
    static __device__ __forceinline__ void issue(const Plan &pl, char *lds, const void *g) {
        const uint32_t l0 = lds_addr(lds) + pl.wave_lds;
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            dma16_sbase(static_cast<const char *>(g) + (i / P) * (P * R * RB), pl.goff[i % P], l0 + i * NTH * 16);
    }
};
// 16-bit rows of D elements.
template <int D, int ROWS, int NTH = NT>
using AsyncTile = AsyncRows<D * 2, ROWS, NTH>;

// The same copy for a tile whose rows sit `stride` bytes apart in global
// memory (a column slice of a wider matrix).
template <int W, int ROWS, int NTH = NT>
struct AsyncTileStrided {
    static constexpr int CH = W / 8;
    static constexpr int LOADS = ROWS * CH / NTH;
    static_assert(ROWS * CH % NTH == 0, "tile not divisible among threads");
    static constexpr int R = NTH / CH;
    static constexpr int P = (R % 16 == 0 || LOADS == 1) ? 1 : (16 / R < LOADS ? 16 / R : LOADS);
    static_assert(R % 16 == 0 || 16 % R == 0, "swizzle period");
    struct Plan {
        uint32_t goff[P];
        uint32_t wave_lds;
    };
    static __device__ __forceinline__ Plan plan(int tid, uint32_t stride) {
        Plan pl;
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const int p = i * NTH + tid, row = p / CH, pc = p % CH;
            const int c = pc ^ swz<CH>(row);
            pl.goff[i] = static_cast<uint32_t>(row) * stride + static_cast<uint32_t>(c * 16);
        }
        pl.wave_lds = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>((tid & ~63) * 16));
        return pl;
    }
    static __device__ __forceinline__ void issue(const Plan &pl, char *lds, const void *g, uint32_t stride) {
        const uint32_t l0 = lds_addr(lds) + pl.wave_lds;
#pragma unroll
        for (int i = 0; i < LOADS; ++i)
            dma16_sbase(static_cast<const char *>(g) + static_cast<size_t>(i / P) * (P * R) * stride, pl.goff[i % P],
                        l0 + i * NTH * 16);
    }
};

// One wave copies 64 consecutive fp32 values (256 bytes) into LDS.
__device__ __forceinline__ void issue_row_stats(float *lds, const float *g, int lane) {
    dma4(g + lane, lds);
}

// s_waitcnt vmcnt(N); a compiler barrier for memory accesses as well.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same value, but the compiler cannot see where it came from: address
// arithmetic derived from it is then done where it is used, not hoisted out
// of enclosing loops (where it would hold registers for the whole loop).
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}
// Forces the wait for a uniform value's loads at this point.
__device__ __forceinline__ void scalar_ready(const int4 &v) {
    asm volatile("" ::"s"(v.x), "s"(v.y), "s"(v.z), "s"(v.w));
}
// Read-only plan arrays through the constant address space: uniform indices
// then become scalar loads, which do not count against vmcnt.
typedef __attribute__((address_space(4))) const int32_t const_i32;
__device__ __forceinline__ const const_i32 *as_const(const int32_t *p) { return (const const_i32 *)p; }
// Barrier that also keeps the compiler from moving LDS accesses across it.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Register fragment of a row-major global matrix row: k0..k0+KL-1.
__device__ __forceinline__ bf16x8 gfrag(const __bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f16x8 gfrag(const _Float16 *p) { return *reinterpret_cast<const f16x8 *>(p); }
__device__ __forceinline__ float gfrag(const float *p) { return *p; }

// Store 4 consecutive output elements converted from fp32.
__device__ __forceinline__ void store4(__bf16 *p, float a, float b, float c, float d) {
    bf16x4 v = {static_cast<__bf16>(a), static_cast<__bf16>(b), static_cast<__bf16>(c), static_cast<__bf16>(d)};
    *reinterpret_cast<bf16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(_Float16 *p, float a, float b, float c, float d) {
    f16x4 v = {static_cast<_Float16>(a), static_cast<_Float16>(b), static_cast<_Float16>(c), static_cast<_Float16>(d)};
    *reinterpret_cast<f16x4 *>(p) = v;
}
__device__ __forceinline__ void store4(float *p, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(p) = make_float4(a, b, c, d);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Combine a value with the one held by the lane 32 apart (v_permlane32_swap,
// no LDS round trip): lanes l and l ^ 32 hold the two halves of a score row.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// acc + sum of the 8 16-bit values of a fragment, two per v_dot2_f32_{bf16,f16}.
__device__ __forceinline__ float rowsum_acc(const f16x8 &f, float acc) {
    const f16x2 one = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f16x2 pr = {f[e], f[e + 1]};
        acc = __builtin_amdgcn_fdot2(pr, one, acc, false);
    }
    return acc;
}
__device__ __forceinline__ float rowsum_acc(const bf16x8 &f, float acc) {
    const bf16x2 one = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 pr = {f[e], f[e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
    return acc;
}

// acc + <a, b> over the elements of two fragments (fp32 products and sums).
__device__ __forceinline__ float frag_dot(const bf16x8 &a, const bf16x8 &b, float acc) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const bf16x2 x = {a[e], a[e + 1]}, y = {b[e], b[e + 1]};
        acc = __builtin_amdgcn_fdot2_f32_bf16(x, y, acc, false);
    }
    return acc;
}
__device__ __forceinline__ float frag_dot(const f16x8 &a, const f16x8 &b, float acc) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
        const f16x2 x = {a[e], a[e + 1]}, y = {b[e], b[e + 1]};
        acc = __builtin_amdgcn_fdot2(x, y, acc, false);
    }
    return acc;
}
__device__ __forceinline__ float frag_dot(float a, float b, float acc) { return fmaf(a, b, acc); }

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Write the accumulator tiles of a wave (lane = output row, values = columns
// 32*dt + 8*(v/4) + 4*(lane/32) + v%4) to a row-major destination row.
// Store a wave's 32 x D bf16 output tile (accumulator layout, lane = row)
// through wave-private LDS scratch of 32 * D * 2 bytes, so that every global
// store writes 16 bytes per lane and 1 KB of consecutive rows per
// instruction. `rows` points at the tile's first row (row stride D). The
// scratch is swizzled by 16-byte chunk (chunk ^ row % 16), which keeps both
// the scattered writes and the row-major reads conflict-free.
template <int D, int DT, typename H>
__device__ __forceinline__ void store_tile_lds(char *scratch, H *rows, const f32x16 (&acc)[DT], float mul,
                                               int lane) {
    typedef __attribute__((ext_vector_type(4))) H h4;
    constexpr int CH = D / 8;  // 16-byte chunks per row
    lane = opaque(lane);
    const int li = lane & 31, lh = lane >> 5;
    auto at = [](int row, int chunk) { return row * (D * 2) + ((chunk ^ (row & 15 & (CH - 1))) << 4); };
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const h4 v = {static_cast<H>(acc[dt][4 * g] * mul), static_cast<H>(acc[dt][4 * g + 1] * mul),
                          static_cast<H>(acc[dt][4 * g + 2] * mul), static_cast<H>(acc[dt][4 * g + 3] * mul)};
            *reinterpret_cast<h4 *>(scratch + at(li, 4 * dt + g) + 8 * lh) = v;
        }
    // LDS operations of one wave complete in order; this only keeps the
    // compiler from moving the reads above the writes of other lanes.
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
#pragma unroll
    for (int i = 0; i < 32 * CH / 64; ++i) {
        const int idx = i * 64 + lane, row = idx / CH, chunk = idx % CH;
        const uint4 v = *reinterpret_cast<const uint4 *>(scratch + at(row, chunk));
        *reinterpret_cast<uint4 *>(rows + static_cast<size_t>(row) * D + chunk * 8) = v;
    }
}

template <int DT, typename OutT>
__device__ __forceinline__ void store_rows(OutT *row, const f32x16 (&acc)[DT], float mul, int lh) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            store4(row + 32 * dt + 8 * g + 4 * lh, acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul,
                   acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul);
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
struct FwdArgs {
    const void *q, *k, *v;
    void *o;
    float *row_max, *row_denom;
    const int4 *items;
    const int32_t *col_idx;
    float *part_o, *part_m2, *part_l, *part_mx;
    int BH, S;
    float c;  // scale * log2(e)
};

// Largest growth of a row's max (base 2) absorbed without rescaling.
constexpr float RESCALE_LOG2 = 8.f;

// Forward modes. ONE_PASS: online softmax, O and statistics in one sweep.
// The two-pass variant (page "trnsparse 0.4.1 -> 0.6.0", CHANGELOG 0.4.3 and
// 0.4.4: a statistics pass, then an output pass that recomputes the scores
// and applies the final row statistics): STATS sweeps the keys for the row
// max and sum only (no V, no P V); OUT recomputes the scores, normalises
// P = 2^(S*c - lse2) with the statistics of the first pass and accumulates
// P V (no running max).
enum FwdMode { FWD_ONE_PASS = 0, FWD_STATS = 1, FWD_OUT = 2 };

template <typename T, int D, int SB, int MINW, int MODE>
__global__ void __launch_bounds__(NT, MINW) fwd_kernel(FwdArgs a) {
    using O = Op<T>;
    using Tl = ATile<T, D>;
    using AT = AsyncRows<D * static_cast<int>(sizeof(T)), SB>;
    constexpr bool B16 = sizeof(T) == 2;
    constexpr int TILE = SB * D * sizeof(T);
    constexpr int NSUB = BLK / SB;    // staged sub-blocks per key block
    constexpr int KS = D / O::KW;     // k-steps along head_dim
    constexpr int NKT = SB / 32;      // 32-key tiles per staged sub-block
    constexpr int KSK = SB / O::KW;   // k-steps along the keys of a sub-block
    constexpr int VPK = 32 / O::KW;   // k-steps per 32-key tile
    constexpr int DT = D / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const int qr = I * BLK + 32 * w + li;  // this lane's query row

    // Running statistics in base-2 units. m2 is the reference the exponentials
    // are taken against; it is raised only when a row's max exceeds it by
    // more than RESCALE_LOG2 (so P <= 2^RESCALE_LOG2 and the accumulator is
    // rescaled rarely). mx2 is the exact running max, returned as row_max.
    float m2 = -INFINITY, mx2 = -INFINITY, lsum = 0.f;
    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

    const int nstage = (p1 - p0) * NSUB;
    const auto tp = AT::plan(tid);
    const const_i32 *cols = as_const(a.col_idx);
    auto first_row = [&](int k) -> size_t {
        return static_cast<size_t>(cols[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
    };
    // Q comes in through LDS when its 128 rows fit one stage buffer: the
    // workgroup's copies are then 1 KB contiguous per instruction, and they
    // overlap the first stage's copies. Otherwise each lane loads its own
    // fragments, after the first stage's copies are issued.
    constexpr bool QLDS = 2 * TILE >= BLK * D * static_cast<int>(sizeof(T));
    if constexpr (QLDS) {
#pragma unroll
        for (int h = 0; h < NSUB; ++h)
            AT::issue(tp, smem + 2 * TILE + h * TILE, Q + static_cast<size_t>(I * BLK + h * SB) * D);
    }
    constexpr int STAGE_TILES = MODE == FWD_STATS ? 1 : 2;  // K only, or K and V
    if (nstage > 0) {
        const size_t r0 = first_row(0);
        AT::issue(tp, smem, K + r0 * D);
        if constexpr (MODE != FWD_STATS) AT::issue(tp, smem + TILE, V + r0 * D);
    }
    typename O::frag qf[KS];
    if constexpr (QLDS) {
        if (nstage > 0) wait_vmcnt<STAGE_TILES * AT::LOADS>();
        else wait_vmcnt<0>();
        barrier_lds();
        const char *qt = smem + 2 * TILE + ((32 * w) / SB) * TILE;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = Tl::frag_row(qt, (32 * w) % SB + li, ks * O::KW + lh * O::KL);
    } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag(Q + static_cast<size_t>(qr) * D + ks * O::KW + lh * O::KL);
    }
    // OUT: the row's base-2 log-sum-exp from the first pass (+inf for an
    // empty row, so that P = 0).
    [[maybe_unused]] float lse = 0.f;
    if constexpr (MODE == FWD_OUT) {
        const size_t sr = static_cast<size_t>(bh) * a.S + qr;
        const float rden = a.row_denom[sr];
        lse = rden > 0.f ? fmaf(a.row_max[sr], LOG2E, log2f(rden)) : INFINITY;
    }

    // One stage: the K (and V) rows of stage k, in stage buffer BUF. Up to
    // head_dim 128 the stage loop below is unrolled by two and BUF
    // is a compile-time constant, so that the LDS addresses of the two
    // buffers differ by an immediate offset and no address arithmetic is
    // repeated per stage (at head_dim 256 the unrolled loop measured 1-2 %
    // slower). FIRST: the row statistics start at this stage (nothing to
    // rescale).
    auto stage = [&](int k, auto buf, auto first_tag) {
        const int BUF = static_cast<int>(buf);
        constexpr bool FIRST = decltype(first_tag)::value;
        char *kt = smem + BUF * 2 * TILE;
        char *vt = kt + TILE;
        // One barrier per stage: after it every wave's copies for this stage
        // are visible and every wave is done with the previous stage, whose
        // buffer the next stage's copies refill.
        wait_vmcnt<0>();
        barrier_lds();
        if (k + 1 < nstage) {
            char *nk = smem + (BUF ^ 1) * 2 * TILE;
            const size_t r1 = first_row(k + 1);
            AT::issue(tp, nk, K + r1 * D);
            if constexpr (MODE != FWD_STATS) AT::issue(tp, nk + TILE, V + r1 * D);
        }

        f32x16 s[NKT];
        if constexpr (B16) {
            // K row operands are read two products ahead of their use, with
            // sched_barrier keeping that order; left to itself the compiler
            // issues each read just before its MFMA and waits for it.
            constexpr int PF = 2, NS = PF + 1, NG = NKT * KS;
            typename O::frag ka[NS];
            auto ld = [&](int g) {
                if (g < NG)
                    ka[g % NS] = Tl::frag_row(kt, 32 * (g / KS) + O::pi(li), (g % KS) * O::KW + lh * O::KL);
            };
#pragma unroll
            for (int t = 0; t < NKT; ++t) s[t] = zero16();
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                ld(g + PF);
                s[g / KS] = O::mma(ka[g % NS], qf[g % KS], s[g / KS]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = zero16();
                const int row = 32 * t + O::pi(li);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    s[t] = O::mma(Tl::frag_row(kt, row, ks * O::KW + lh * O::KL), qf[ks], s[t]);
            }
        }
        if constexpr (MODE == FWD_OUT) {
            if constexpr (D > 256) {
                // At head_dim 512 the accumulator takes 256 registers: the
                // transposed V operands go through a three-slot ring, read two
                // products ahead (left to itself the compiler reads all of a
                // stage's at once and spills).
                typename O::frag pfs[KSK];
#pragma unroll
                for (int kk = 0; kk < KSK; ++kk) {
                    f32x16 &st = s[kk / VPK];
#pragma unroll
                    for (int e = 0; e < O::KL; ++e) {
                        const int v = (kk % VPK) * O::KL + e;
                        st[v] = exp2_fast(fmaf(st[v], a.c, -lse));
                    }
                    pfs[kk] = O::pack(st, (kk % VPK) * O::KL);
                }
                constexpr int PF = 2, NS = PF + 1, NG = KSK * DT;
                typename O::frag vb[NS];
                auto ld = [&](int g) {
                    if (g < NG) vb[g % NS] = Tl::frag_tr(vt, (g / DT) * O::KW, 32 * (g % DT), lane);
                };
#pragma unroll
                for (int g = 0; g < PF; ++g) ld(g);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    ld(g + PF);
                    acc[g % DT] = O::mma(vb[g % NS], pfs[g / DT], acc[g % DT]);
                    __builtin_amdgcn_sched_barrier(0);
                }
                return;
            }
#pragma unroll
            for (int kk = 0; kk < KSK; ++kk) {
                typename O::frag pf;
                {
                    f32x16 &st = s[kk / VPK];
#pragma unroll
                    for (int e = 0; e < O::KL; ++e) {
                        const int v = (kk % VPK) * O::KL + e;
                        st[v] = exp2_fast(fmaf(st[v], a.c, -lse));
                    }
                    pf = O::pack(st, (kk % VPK) * O::KL);
                }
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    acc[dt] = O::mma(Tl::frag_tr(vt, kk * O::KW, 32 * dt, lane), pf, acc[dt]);
            }
            return;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[t][v]);
        mx = pair_max(mx) * a.c;
        mx2 = fmaxf(mx2, mx);
        if constexpr (FIRST) {
            m2 = mx;  // the accumulator and the sum are still zero
        } else if (mx > m2 + RESCALE_LOG2) {  // per row; skipped by whole waves when no row needs it
            const float corr = exp2_fast(m2 - mx);
            lsum *= corr;
            if constexpr (MODE == FWD_ONE_PASS) {
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[dt][v] *= corr;
            }
            m2 = mx;
        }
        float rs = 0.f;
        if constexpr (MODE == FWD_STATS) {  // fp32 sum of the exponentials: the exact statistic
#pragma unroll
            for (int t = 0; t < NKT; ++t)
#pragma unroll
                for (int v = 0; v < 16; ++v) rs += exp2_fast(fmaf(s[t][v], a.c, -m2));
            lsum += pair_sum(rs);
            return;
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                s[t][v] = exp2_fast(fmaf(s[t][v], a.c, -m2));
                if constexpr (!B16) rs += s[t][v];
            }
#pragma unroll
        for (int kk = 0; kk < KSK; ++kk) {
            const typename O::frag pf = O::pack(s[kk / VPK], (kk % VPK) * O::KL);
            // bf16: the row sum is taken over the rounded P the product uses
            if constexpr (B16) rs = rowsum_acc(pf, rs);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc[dt] = O::mma(Tl::frag_tr(vt, kk * O::KW, 32 * dt, lane), pf, acc[dt]);
        }
        lsum += pair_sum(rs);
    };
    using B0 = std::integral_constant<int, 0>;
    using B1 = std::integral_constant<int, 1>;
    using F1 = std::true_type;
    using F0 = std::false_type;
    if (nstage > 0) stage(0, B0{}, F1{});
    if constexpr (D <= 128) {
        for (int k = 1; k < nstage; k += 2) {
            stage(k, B1{}, F0{});
            if (k + 1 < nstage) stage(k + 1, B0{}, F0{});
        }
    } else {
        for (int k = 1; k < nstage; ++k) stage(k, k & 1, F0{});
    }

    const size_t srow = static_cast<size_t>(bh) * a.S + qr;
    if constexpr (MODE == FWD_STATS) {
        if (lh == 0) {
            if (slot < 0) {
                a.row_max[srow] = lsum > 0.f ? mx2 / LOG2E : -INFINITY;
                a.row_denom[srow] = lsum > 0.f ? lsum * exp2_fast(m2 - mx2) : 0.f;
            } else {
                const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
                a.part_m2[prow] = m2;
                a.part_l[prow] = lsum;
                a.part_mx[prow] = mx2;
            }
        }
        return;
    }
    if constexpr (MODE == FWD_OUT) {  // P was normalised: the sum is O (or its share)
        if (slot < 0) {
            if constexpr (B16 && 4 * 32 * D * 2 <= 2 * TILE) {
                char *scratch = smem + (nstage & 1) * 2 * TILE + w * (32 * D * 2);
                store_tile_lds<D, DT>(scratch,
                                      static_cast<T *>(a.o) + base + static_cast<size_t>(I * BLK + 32 * w) * D, acc,
                                      1.f, lane);
            } else {
                store_rows<DT>(static_cast<T *>(a.o) + base + static_cast<size_t>(qr) * D, acc, 1.f, lh);
            }
        } else {
            const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
            store_rows<DT>(a.part_o + prow * D, acc, 1.f, lh);
        }
        return;
    }
    if (slot < 0) {
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
        if constexpr (B16 && 4 * 32 * D * 2 <= 2 * TILE) {
            // the buffer the last stage did not read is free for every wave
            char *scratch = smem + (nstage & 1) * 2 * TILE + w * (32 * D * 2);
            store_tile_lds<D, DT>(scratch, static_cast<T *>(a.o) + base + static_cast<size_t>(I * BLK + 32 * w) * D,
                                  acc, inv, lane);
        } else {
            store_rows<DT>(static_cast<T *>(a.o) + base + static_cast<size_t>(qr) * D, acc, inv, lh);
        }
        if (lh == 0) {
            a.row_max[srow] = lsum > 0.f ? mx2 / LOG2E : -INFINITY;
            a.row_denom[srow] = lsum > 0.f ? lsum * exp2_fast(m2 - mx2) : 0.f;
        }
    } else {
        const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
        store_rows<DT>(a.part_o + prow * D, acc, 1.f, lh);
        if (lh == 0) {
            a.part_m2[prow] = m2;
            a.part_l[prow] = lsum;
            a.part_mx[prow] = mx2;
        }
    }
}

struct MergeArgs {
    const int4 *merges;
    const float *part_o, *part_m2, *part_l, *part_mx;
    void *o;
    float *row_max, *row_denom;
    int BH, S;
};

// Merges and partial sums give each thread one 4-column chunk of one row:
// NT / (D / 4) rows per workgroup, D / 8 workgroups per 128-row line.
template <int D> constexpr int merge_slices() { return BLK / (NT / (D / 4)); }

// Log-sum-exp merge of split rows: m = max m_s, l = sum l_s 2^(m_s - m),
// O = sum O_s 2^(m_s - m) / l, with (m_s, l_s) each segment's reference and
// sum in base-2 units, taken in one pass with a running reference so that
// the loads of every segment are independent of the arithmetic. The
// returned row_max is the largest segment max and row_denom is l
// re-expressed against it. One workgroup per (merge, batch*head, slice).
template <typename T, int D, bool WITH_O>
__global__ void __launch_bounds__(NT) fwd_merge_kernel(MergeArgs a) {
    constexpr int CH = D / 4;
    constexpr int MR = NT / CH;
    constexpr int SLICES = merge_slices<D>();
    const int slice = blockIdx.x % SLICES;
    const int bh = (blockIdx.x / SLICES) % a.BH;
    const int mi = blockIdx.x / SLICES / a.BH;
    const int4 mg = a.merges[mi];
    const int I = mg.x, s0 = mg.y, ns = mg.z;
    const int r = slice * MR + threadIdx.x / CH, c = threadIdx.x % CH;
    // Every segment holds at least one block, so each m_s is finite.
    float m = -INFINITY, l = 0.f, mx = -INFINITY;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
        const size_t pr = (static_cast<size_t>(s0 + s) * a.BH + bh) * BLK + r;
        const float ms = a.part_m2[pr], ls = a.part_l[pr];
        const float4 x = WITH_O ? *reinterpret_cast<const float4 *>(a.part_o + pr * D + 4 * c)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        mx = fmaxf(mx, a.part_mx[pr]);
        const float mn = fmaxf(m, ms);
        const float co = exp2_fast(m - mn), cs = exp2_fast(ms - mn);
        l = fmaf(l, co, ls * cs);
        acc.x = fmaf(acc.x, co, x.x * cs);
        acc.y = fmaf(acc.y, co, x.y * cs);
        acc.z = fmaf(acc.z, co, x.z * cs);
        acc.w = fmaf(acc.w, co, x.w * cs);
        m = mn;
    }
    const float inv = 1.f / l;
    const size_t srow = static_cast<size_t>(bh) * a.S + I * BLK + r;
    if constexpr (WITH_O)
        store4(static_cast<T *>(a.o) + srow * D + 4 * c, acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
    if (c == 0) {
        a.row_max[srow] = mx / LOG2E;
        a.row_denom[srow] = l * exp2_fast(m - mx);
    }
}

struct DqArgs {
    const void *q, *k, *v, *o, *dout;
    const float *row_max, *row_denom;
    float *delta, *lse2;  // written here for the dK/dV pass (delta negated: -D)
    void *dq;
    const int4 *items;
    const int32_t *col_idx, *row_ptr;
    float *part;
    int BH, S;
    float c, scale;
};

// Row-first dQ: for each stored block J of the row,
//   S^T = K_J Q^T, dP^T = V_J dO^T, P = 2^(S*c - lse2), dS = P (dP - delta),
//   dQ^T += K_J^T dS^T;  dQ = scale * dQ.
// The row terms are formed in the prologue: delta = <dO_r, O_r> over the
// returned O, lse2 = row_max * log2(e) + log2(row_denom) (+inf for an empty
// row, which makes P = 0). The workgroup holding the first segment of the
// row also stores them for the dK/dV pass.
template <typename T, int D, int SB, int MINW>
__global__ void __launch_bounds__(NT, MINW) dq_kernel(DqArgs a) {
    using O = Op<T>;
    using Tl = ATile<T, D>;
    using AT = AsyncRows<D * static_cast<int>(sizeof(T)), SB>;
    constexpr bool B16 = sizeof(T) == 2;
    constexpr int TILE = SB * D * sizeof(T);
    constexpr int NSUB = BLK / SB;
    constexpr int KS = D / O::KW;
    constexpr int NKT = SB / 32;
    constexpr int KSK = SB / O::KW;
    constexpr int VPK = 32 / O::KW;
    constexpr int DT = D / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const T *dO = static_cast<const T *>(a.dout) + base;
    const T *Ob = static_cast<const T *>(a.o) + base;
    const int qr = I * BLK + 32 * w + li;
    const size_t srow = static_cast<size_t>(bh) * a.S + qr;

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

    const int nstage = (p1 - p0) * NSUB;
    const auto tp = AT::plan(tid);
    const const_i32 *cols = as_const(a.col_idx);
    auto first_row = [&](int k) -> size_t {
        return static_cast<size_t>(cols[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
    };
    if (nstage > 0) {
        const size_t r0 = first_row(0);
        AT::issue(tp, smem, K + r0 * D);
        AT::issue(tp, smem + TILE, V + r0 * D);
    }
    typename O::frag qf[KS], df[KS];
    float dlt = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const size_t off = static_cast<size_t>(qr) * D + ks * O::KW + lh * O::KL;
        qf[ks] = gfrag(Q + off);
        df[ks] = gfrag(dO + off);
        dlt = frag_dot(gfrag(Ob + off), df[ks], dlt);
    }
    dlt = pair_sum(dlt);
    const float rden = a.row_denom[srow];
    const float lse = rden > 0.f ? fmaf(a.row_max[srow], LOG2E, log2f(rden)) : INFINITY;
    if (lh == 0 && (slot < 0 || p0 == as_const(a.row_ptr)[I])) {
        a.delta[srow] = -dlt;  // stored negated (see dkdv_pair_kernel)
        a.lse2[srow] = lse;
    }

    // One stage in buffer BUF. Up to head_dim 128 the loop below is unrolled
    // by two and BUF is a compile-time index: LDS addresses of the two
    // buffers then differ by an immediate offset, with no address arithmetic
    // per stage. (At head_dim 256 the unrolled loop spills registers.)
    auto stage = [&](int k, auto buf) {
        const int BUF = static_cast<int>(buf);
        char *kt = smem + BUF * 2 * TILE;
        char *vt = kt + TILE;
        // One barrier per stage: after it every wave's copies for this stage
        // are visible and every wave is done with the previous stage, whose
        // buffer the next stage's copies refill.
        wait_vmcnt<0>();
        barrier_lds();
        if (k + 1 < nstage) {
            char *nk = smem + (BUF ^ 1) * 2 * TILE;
            const size_t r1 = first_row(k + 1);
            AT::issue(tp, nk, K + r1 * D);
            AT::issue(tp, nk + TILE, V + r1 * D);
        }

        // dP - delta in one accumulation: the products start from -delta
        auto ndl16 = [&] {
            f32x16 z;
#pragma unroll
            for (int v = 0; v < 16; ++v) z[v] = -dlt;
            return z;
        };
        f32x16 s[NKT], dp[NKT];
        if constexpr (B16 || D >= 128) {
            // The K and V row operands of the score products are read two
            // products ahead of their use; sched_barrier keeps the compiler
            // from sinking each read next to its MFMA, where the MFMA would
            // wait out the LDS latency (measured, same results bit for bit:
            // dQ 8 % faster on the bf16 global-mask workload, 10 % on fp32
            // random 10 % at head_dim 128, 5 % slower on fp32 at head_dim 64;
            // in the fp32 forward the same order measured three times
            // slower, so the forward keeps it to 16-bit operands).
            constexpr int PF = 2, NS = PF + 1, NG = NKT * KS;
            typename O::frag ka[NS], va[NS];
            auto ld = [&](int g) {
                if (g < NG) {
                    const int row = 32 * (g / KS) + O::pi(li), ks = g % KS;
                    ka[g % NS] = Tl::frag_row(kt, row, ks * O::KW + lh * O::KL);
                    va[g % NS] = Tl::frag_row(vt, row, ks * O::KW + lh * O::KL);
                }
            };
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = zero16();
                dp[t] = ndl16();
            }
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                ld(g + PF);
                const int t = g / KS, ks = g % KS;
                s[t] = O::mma(ka[g % NS], qf[ks], s[t]);
                dp[t] = O::mma(va[g % NS], df[ks], dp[t]);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int t = 0; t < NKT; ++t) {
                s[t] = zero16();
                dp[t] = ndl16();
                const int row = 32 * t + O::pi(li);
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    s[t] = O::mma(Tl::frag_row(kt, row, ks * O::KW + lh * O::KL), qf[ks], s[t]);
                    dp[t] = O::mma(Tl::frag_row(vt, row, ks * O::KW + lh * O::KL), df[ks], dp[t]);
                }
            }
        }
#pragma unroll
        for (int t = 0; t < NKT; ++t)
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const float p = exp2_fast(fmaf(s[t][v], a.c, -lse));
                s[t][v] = p * dp[t][v];  // dp holds dP - delta
            }
#pragma unroll
        for (int kk = 0; kk < KSK; ++kk) {
            const typename O::frag bf = O::pack(s[kk / VPK], (kk % VPK) * O::KL);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
                acc[dt] = O::mma(Tl::frag_tr(kt, kk * O::KW, 32 * dt, lane), bf, acc[dt]);
        }
    };
    if constexpr (D <= 128) {
        for (int k = 0; k < nstage; k += 2) {
            stage(k, std::integral_constant<int, 0>{});
            if (k + 1 < nstage) stage(k + 1, std::integral_constant<int, 1>{});
        }
    } else {
        for (int k = 0; k < nstage; ++k) stage(k, k & 1);
    }

    if (slot < 0) {
        if constexpr (B16 && 4 * 32 * D * 2 <= 2 * TILE) {
            char *scratch = smem + (nstage & 1) * 2 * TILE + w * (32 * D * 2);
            store_tile_lds<D, DT>(scratch, static_cast<T *>(a.dq) + base + static_cast<size_t>(I * BLK + 32 * w) * D,
                                  acc, a.scale, lane);
        } else {
            store_rows<DT>(static_cast<T *>(a.dq) + base + static_cast<size_t>(qr) * D, acc, a.scale, lh);
        }
    } else {
        const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
        store_rows<DT>(a.part + prow * D, acc, a.scale, lh);
    }
}

struct DkdvArgs {
    const void *q, *k, *v, *dout;
    const float *delta, *lse2;
    void *dk, *dv;
    const int4 *items;
    const int32_t *row_idx;
    const int32_t *queues;  // schedule for n_queues work queues per head
    float *part_dk, *part_dv;
    int BH, S, n_queues;
    float c, scale;
    // dS-storing variant: dS^T blocks [BH][nnzb][128 keys][128 queries] in
    // the operand dtype, indexed by BSR position (bsc_block maps the BSC
    // entries the pass walks to it).
    void *ds;
    const int32_t *bsc_block;
    int nnzb;
};

// One staged sub-block of the dK/dV pass: SB query rows of Q and dO (qt, ot)
// with their lse2 and delta (sl, sd) against the wave's 32 keys (kf, vf).
//
// DS: also store the stage's dS (as rounded for the dK product) to `ds`, the
// lane's key row of the block's dS^T at the stage's first query. With the pi
// row order, the two packed fragments of a 32-query tile are queries
// 32t + 16kk + 8*(lane/32) + 0..7 of that row: one 16-byte store each.
template <typename T, int D, int SB, bool DS = false>
__device__ __forceinline__ void dkdv_stage(const char *qt, const char *ot, const float *sl, const float *sd,
                                           const typename Op<T>::frag (&kf)[D / Op<T>::KW],
                                           const typename Op<T>::frag (&vf)[D / Op<T>::KW], f32x16 (&dk)[D / 32],
                                           f32x16 (&dv)[D / 32], float c, int lane, T *ds = nullptr) {
    static_assert(!DS || sizeof(T) == 2, "dS is stored for 16-bit operands only");
    static_assert(sizeof(T) == 4 || D <= 128, "16-bit head_dim 256 runs in dkdv_wide_pair_kernel");
    using O = Op<T>;
    using Tl = ATile<T, D>;
    constexpr int KS = D / O::KW;
    constexpr int NQT = SB / 32;     // 32-query tiles per staged sub-block
    constexpr int VPK = 32 / O::KW;  // k-steps per 32-query tile
    constexpr int DT = D / 32;
    const int li = lane & 31, lh = lane >> 5;
    // Query tiles are processed one at a time: unrolling or software-pipelining
    // them measured slower on gfx950 (register pressure, no gain in overlap).
#pragma unroll 1
    for (int t = 0; t < NQT; ++t) {
        f32x16 s = zero16(), dp = zero16();
        const int row = 32 * t + O::pi(li);
        if constexpr (sizeof(T) == 2) {
            // Q and dO row operands are read two products ahead of their
            // use, with sched_barrier keeping that order: left to itself the
            // compiler issues each read just before its MFMA, and at one wave
            // per SIMD nothing covers the LDS latency (measured: dK/dV 2 %
            // faster on the global-mask workload, same results bit for bit).
            constexpr int PF = 2, NSL = PF + 1;
            typename O::frag qa[NSL], oa[NSL];
            auto ld = [&](int ks) {
                if (ks < KS) {
                    qa[ks % NSL] = Tl::frag_row(qt, row, ks * O::KW + lh * O::KL);
                    oa[ks % NSL] = Tl::frag_row(ot, row, ks * O::KW + lh * O::KL);
                }
            };
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ld(ks + PF);
                s = O::mma(qa[ks % NSL], kf[ks], s);
                dp = O::mma(oa[ks % NSL], vf[ks], dp);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                s = O::mma(Tl::frag_row(qt, row, ks * O::KW + lh * O::KL), kf[ks], s);
                dp = O::mma(Tl::frag_row(ot, row, ks * O::KW + lh * O::KL), vf[ks], dp);
            }
        }
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int qi = 32 * t + O::pi(8 * (v >> 2) + 4 * lh + (v & 3));
            const float p = exp2_fast(fmaf(s[v], c, -sl[qi]));
            s[v] = p;
            dp[v] = p * (dp[v] + sd[qi]);
        }
#pragma unroll
        for (int kk = 0; kk < VPK; ++kk) {
            const typename O::frag bp = O::pack(s, kk * O::KL);
            const typename O::frag bd = O::pack(dp, kk * O::KL);
            if constexpr (DS) *reinterpret_cast<typename O::frag *>(ds + 32 * t + 16 * kk + 8 * lh) = bd;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
                dv[dt] = O::mma(Tl::frag_tr(ot, 32 * t + kk * O::KW, 32 * dt, lane), bp, dv[dt]);
                dk[dt] = O::mma(Tl::frag_tr(qt, 32 * t + kk * O::KW, 32 * dt, lane), bd, dk[dt]);
            }
        }
    }
}

// Column-first dK/dV (fp32 operands; the 16-bit instances run in the queue
// and pair kernels): the workgroup owns 128 keys of block column J; for each
// block row I that stores J (BSC order), in 32-query tiles:
//   S = Q_t K^T, dP = dO_t V^T, P = 2^(S*c - lse2), dS = P (dP - delta),
//   dV^T += dO_t^T P, dK^T += Q_t^T dS;  dK = scale * dK.
template <typename T, int D, int SB, int MINW>
__global__ void __launch_bounds__(NT, MINW) dkdv_kernel(DkdvArgs a) {
    using O = Op<T>;
    using AT = AsyncRows<D * static_cast<int>(sizeof(T)), SB>;
    static_assert(sizeof(T) == 4, "fp32 operands");
    constexpr int TILE = SB * D * sizeof(T);
    constexpr int NSUB = BLK / SB;
    constexpr int KS = D / O::KW;
    constexpr int DT = D / 32;
    static_assert(SB == 64 || SB == 128, "row statistics are staged by whole waves");
    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float s_lse[2][SB], s_dlt[2][SB];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int J = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const T *dO = static_cast<const T *>(a.dout) + base;
    const float *LSE = a.lse2 + static_cast<size_t>(bh) * a.S;
    const float *DLT = a.delta + static_cast<size_t>(bh) * a.S;
    const int kr = J * BLK + 32 * w + li;  // this lane's key row

    f32x16 dk[DT], dv[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
        dk[dt] = zero16();
        dv[dt] = zero16();
    }

    const int nstage = (p1 - p0) * NSUB;
    const auto tp = AT::plan(tid);
    const const_i32 *rows = as_const(a.row_idx);
    auto first_row = [&](int k) -> size_t {
        return static_cast<size_t>(rows[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
    };
    // Row statistics of a stage: SB/64 wave-loads each of lse2 and delta.
    // SB == 128: waves 0,1 load lse2 halves, waves 2,3 delta halves (one each);
    // SB == 64: wave 0 loads lse2, wave 1 delta.
    auto issue_stats = [&](int buf, size_t r0) {
        if constexpr (SB == 128) {
            const int half = w & 1;
            if (w < 2) issue_row_stats(&s_lse[buf][64 * half], LSE + r0 + 64 * half, lane);
            else issue_row_stats(&s_dlt[buf][64 * half], DLT + r0 + 64 * half, lane);
        } else {
            if (w == 0) issue_row_stats(&s_lse[buf][0], LSE + r0, lane);
            else if (w == 1) issue_row_stats(&s_dlt[buf][0], DLT + r0, lane);
        }
    };
    if (nstage > 0) {
        const size_t r0 = first_row(0);
        AT::issue(tp, smem, Q + r0 * D);
        AT::issue(tp, smem + TILE, dO + r0 * D);
        issue_stats(0, r0);
    }
    typename O::frag kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = gfrag(K + static_cast<size_t>(kr) * D + ks * O::KW + lh * O::KL);
        vf[ks] = gfrag(V + static_cast<size_t>(kr) * D + ks * O::KW + lh * O::KL);
    }
    for (int k = 0; k < nstage; ++k) {
        const int buf = k & 1;
        char *qt = smem + buf * 2 * TILE;
        char *ot = qt + TILE;
        wait_vmcnt<0>();
        barrier_lds();
        if (k + 1 < nstage) {
            const int nb = buf ^ 1;
            char *nq = smem + nb * 2 * TILE;
            const size_t r1 = first_row(k + 1);
            AT::issue(tp, nq, Q + r1 * D);
            AT::issue(tp, nq + TILE, dO + r1 * D);
            issue_stats(nb, r1);
        }
        dkdv_stage<T, D, SB>(qt, ot, s_lse[buf], s_dlt[buf], kf, vf, dk, dv, a.c, lane);
    }

    if (slot < 0) {
        store_rows<DT>(static_cast<T *>(a.dk) + base + static_cast<size_t>(kr) * D, dk, a.scale, lh);
        store_rows<DT>(static_cast<T *>(a.dv) + base + static_cast<size_t>(kr) * D, dv, 1.f, lh);
    } else {
        const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
        store_rows<DT>(a.part_dk + prow * D, dk, a.scale, lh);
        store_rows<DT>(a.part_dv + prow * D, dv, 1.f, lh);
    }
}

// Column-first dK/dV, persistent form (bf16, head_dim <= 128): the grid is
// n_queues workgroups per (batch*head); workgroup (q, bh) walks the column
// items of work queue q in order. Stages are whole 128-row blocks, double
// buffered. During the last stage of an item the next item's K and V rows go
// into the free buffer; after it, the next item's first stage is issued into
// the other buffer before the current item's outputs are stored, so item
// boundaries overlap copies with work instead of waiting on them. The K/V
// fragments come from LDS (each wave reads its own 32 rows), and each wave
// then uses those same rows of LDS to stage its output tile.
template <typename T, int D, bool DS = false>
__global__ void __launch_bounds__(NT, 1) dkdv_queue_kernel(DkdvArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, D>;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int SB = BLK;
    constexpr int TILE = SB * D * sizeof(T);  // one 128-row tile
    constexpr int KS = D / O::KW;
    constexpr int DT = D / 32;
    constexpr int LOADS = AsyncTile<D, SB>::LOADS;
    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float s_lse[2][SB], s_dlt[2][SB];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int queue = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const const_i32 *qs = as_const(a.queues);
    const int e0 = qs[queue], e1 = qs[queue + 1];
    if (e0 == e1) return;  // whole workgroup: nothing queued
    const const_i32 *qitems = qs + a.n_queues + 1;
    const const_i32 *items = as_const(reinterpret_cast<const int32_t *>(a.items));
    const const_i32 *rows = as_const(a.row_idx);
    auto item = [&](int e) -> int4 {
        const int i = qitems[e];
        return make_int4(items[4 * i], items[4 * i + 1], items[4 * i + 2], items[4 * i + 3]);
    };

    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const T *dO = static_cast<const T *>(a.dout) + base;
    const float *LSE = a.lse2 + static_cast<size_t>(bh) * a.S;
    const float *DLT = a.delta + static_cast<size_t>(bh) * a.S;
    const auto tp = AsyncTile<D, SB>::plan(tid);
    auto buffer = [&](int b) { return smem + b * 2 * TILE; };
    // K and V rows of block column J into buffer b.
    auto issue_kv = [&](int b, int J) {
        AsyncTile<D, SB>::issue(tp, buffer(b), K + static_cast<size_t>(J) * BLK * D);
        AsyncTile<D, SB>::issue(tp, buffer(b) + TILE, V + static_cast<size_t>(J) * BLK * D);
    };
    // Q, dO, lse2 and delta of block row I into buffer b (waves 0, 1: lse2
    // halves; waves 2, 3: delta halves).
    auto issue_stage = [&](int b, int I) {
        const size_t r0 = static_cast<size_t>(I) * BLK;
        AsyncTile<D, SB>::issue(tp, buffer(b), Q + r0 * D);
        AsyncTile<D, SB>::issue(tp, buffer(b) + TILE, dO + r0 * D);
        const int half = w & 1;
        if (w < 2) issue_row_stats(&s_lse[b][64 * half], LSE + r0 + 64 * half, lane);
        else issue_row_stats(&s_dlt[b][64 * half], DLT + r0 + 64 * half, lane);
    };
    // This wave's 32 rows of the K / V tiles held in buffer b.
    auto load_frags = [&](int b, typename O::frag (&kf)[KS], typename O::frag (&vf)[KS]) {
        const int ln = opaque(lane), row = 32 * w + (ln & 31), k0 = (ln >> 5) * O::KL;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            kf[ks] = Tl::frag_row(buffer(b), row, ks * O::KW + k0);
            vf[ks] = Tl::frag_row(buffer(b) + TILE, row, ks * O::KW + k0);
        }
    };

    // First item: its K/V into buffer 1, its first stage into buffer 0.
    int e = e0;
    int4 cur = item(e);
    issue_kv(1, cur.x);
    if (cur.z > cur.y) {
        issue_stage(0, rows[cur.y]);
        wait_vmcnt<2 * LOADS + 1>();
    } else {
        wait_vmcnt<0>();
    }
    barrier_lds();
    typename O::frag kf[KS], vf[KS];
    load_frags(1, kf, vf);
    int sb = 0;  // buffer holding the current item's first stage

    for (;;) {
        const int nstage = cur.z - cur.y;
        const bool more = e + 1 < e1;
        const int4 nxt = more ? item(e + 1) : make_int4(0, 0, 0, 0);
        // Take delivery of these scalar loads now: a scalar load left in
        // flight would make the compiler wait for every LDS read in the stage
        // loop with lgkmcnt(0), since both share that counter.
        scalar_ready(nxt);
        f32x16 dk[DT], dv[DT];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
            dk[dt] = zero16();
            dv[dt] = zero16();
        }
        if (nstage == 0 && more) issue_kv(sb, nxt.x);
        for (int k = 0; k < nstage; ++k) {
            const int b = sb ^ (k & 1);
            wait_vmcnt<0>();
            barrier_lds();  // this stage visible; every wave done with the other buffer
            if (k + 1 < nstage) issue_stage(b ^ 1, rows[cur.y + k + 1]);
            else if (more) issue_kv(b ^ 1, nxt.x);
            T *dsr = nullptr;
            if constexpr (DS) {
                const int blk = as_const(a.bsc_block)[cur.y + k];
                asm volatile("" ::"s"(blk));  // take the scalar load now (see scalar_ready)
                dsr = static_cast<T *>(a.ds) +
                      ((static_cast<size_t>(bh) * a.nnzb + blk) * BLK + 32 * w + opaque(lane & 31)) * BLK;
            }
            dkdv_stage<T, D, SB, DS>(buffer(b), buffer(b) + TILE, s_lse[b], s_dlt[b], kf, vf, dk, dv, a.c, lane,
                                     dsr);
        }
        const int F = sb ^ (nstage & 1);  // free buffer; holds the next K/V when there is a next item
        if (more) {
            wait_vmcnt<0>();
            barrier_lds();  // next K/V visible; every wave done with the last stage's buffer
            if (nxt.z > nxt.y) issue_stage(F ^ 1, rows[nxt.y]);
            load_frags(F, kf, vf);
        }
        // Outputs. Each wave stages through its own 32 rows of the K and V
        // tiles in buffer F (already read into registers above, and read by no
        // other wave).
        const int J = cur.x, slot = cur.w;
        const size_t r0 = static_cast<size_t>(J * BLK + 32 * w) * D;
        if (slot < 0) {
            char *sk = buffer(F) + 32 * w * D * 2;
            // LDS accesses of one wave complete in order: the fragment reads
            // above are served before these writes reach the same rows.
            __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
            store_tile_lds<D, DT>(sk, static_cast<T *>(a.dk) + base + r0, dk, a.scale, lane);
            store_tile_lds<D, DT>(sk + TILE, static_cast<T *>(a.dv) + base + r0, dv, 1.f, lane);
        } else {
            const int ln = opaque(lane);
            const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + (ln & 31);
            store_rows<DT>(a.part_dk + prow * D, dk, a.scale, ln >> 5);
            store_rows<DT>(a.part_dv + prow * D, dv, 1.f, ln >> 5);
        }
        if (!more) break;
        ++e;
        cur = nxt;
        sb = F ^ 1;
    }
}

// Column-first dK/dV with two waves per SIMD (bf16/fp16, head_dim 128): 512
// threads; the two waves that own the same 32 keys of the block column split
// the work of each 32-query tile by role, so that each holds one accumulator
// tile instead of two:
//   role 0 (waves 0-3):  S = Q_t K^T, P = 2^(S*c - lse2), dV^T += dO_t^T P;
//                        P goes to LDS in the packed form the dV product uses;
//   role 1 (waves 4-7):  dP - delta = dO_t V^T accumulated onto -delta (the
//                        row terms are stored negated for this); after the
//                        tile's barrier reads P, dS = P (dP - delta),
//                        dK^T += Q_t^T dS.
// Role 1 finishes tile t (dS, dK) while role 0 works on tile t + 1, so both
// issue 16 products between consecutive barriers and the two waves of a SIMD
// cover each other's softmax work and LDS waits. P is exchanged through a
// double buffer, one barrier per tile. The walk over the column items of a
// work queue, the double-buffered 128-row stages and the item boundaries are
// those of dkdv_queue_kernel; a stage's buffer is refilled only after the
// barrier that ends role 1's last tile of the previous stage, and its copies
// are waited for before the barrier that precedes its first tile. Only the
// role-0 waves issue the LDS-DMA copies (each twice as many): role-1 waves
// then never queue behind the address unit, and the MFMA pipe of each SIMD
// keeps a wave to serve while its partner issues (dK/dV 3-4 % faster than
// all eight waves issuing, bit-identical).
// (dS here is formed from P as rounded for the dV product.)
constexpr int NT2 = 512;

template <typename T, int D, bool DS = false>
__global__ void __launch_bounds__(NT2, 1) dkdv_pair_kernel(DkdvArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, D>;
    using frag = typename O::frag;
    using AT = AsyncTile<D, BLK, NT>;  // copies issued by the 256 role-0 threads
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int TILE = BLK * D * sizeof(T);  // one 128-row tile
    constexpr int KS = D / O::KW;
    constexpr int DT = D / 32;
    constexpr int VPK = 32 / O::KW;
    __shared__ __attribute__((aligned(16))) char smem[2 * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float s_lse[2][BLK], s_dlt[2][BLK];
    __shared__ __attribute__((aligned(16))) frag s_p[2][4][VPK][64];  // [tile parity][pair][k-step][lane]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & 3, role = w >> 2;
    const int li = lane & 31, lh = lane >> 5;
    const int queue = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const const_i32 *qs = as_const(a.queues);
    const int e0 = qs[queue], e1 = qs[queue + 1];
    if (e0 == e1) return;  // whole workgroup: nothing queued
    const const_i32 *qitems = qs + a.n_queues + 1;
    const const_i32 *items = as_const(reinterpret_cast<const int32_t *>(a.items));
    const const_i32 *rows = as_const(a.row_idx);
    auto item = [&](int e) -> int4 {
        const int i = qitems[e];
        return make_int4(items[4 * i], items[4 * i + 1], items[4 * i + 2], items[4 * i + 3]);
    };

    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const T *dO = static_cast<const T *>(a.dout) + base;
    const float *LSE = a.lse2 + static_cast<size_t>(bh) * a.S;
    const float *DLT = a.delta + static_cast<size_t>(bh) * a.S;
    const auto tp = AT::plan(tid & (NT - 1));
    auto buffer = [&](int b) { return smem + b * 2 * TILE; };
    // Copies, issued by the role-0 waves only (role-1 waves return).
    auto issue_kv = [&](int b, int J) {
        if (role) return;
        AT::issue(tp, buffer(b), K + static_cast<size_t>(J) * BLK * D);
        AT::issue(tp, buffer(b) + TILE, V + static_cast<size_t>(J) * BLK * D);
    };
    // Q, dO, lse2 and delta of block row I into buffer b (waves 0, 1: lse2
    // halves; waves 2, 3: delta halves).
    auto issue_stage = [&](int b, int I) {
        if (role) return;
        const size_t r0 = static_cast<size_t>(I) * BLK;
        AT::issue(tp, buffer(b), Q + r0 * D);
        AT::issue(tp, buffer(b) + TILE, dO + r0 * D);
        const int half = w & 1;
        if (w < 2) issue_row_stats(&s_lse[b][64 * half], LSE + r0 + 64 * half, lane);
        else issue_row_stats(&s_dlt[b][64 * half], DLT + r0 + 64 * half, lane);
    };
    // This wave's 32 rows of the K tile (role 0) or the V tile (role 1) in buffer b.
    auto load_frags = [&](int b, frag (&f)[KS]) {
        const int ln = opaque(lane), row = 32 * pair + (ln & 31), k0 = (ln >> 5) * O::KL;
        const char *src = buffer(b) + role * TILE;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) f[ks] = Tl::frag_row(src, row, ks * O::KW + k0);
    };
    // The 16 row statistics of a lane in a 32-query tile: value v belongs to
    // query 32t + 16(a/2) + 8(lane/32) + 4(a%2) + v%4, a = v/4 (the pi row
    // order), four runs of four consecutive queries.
    auto stats = [&](const float *st, int t, float (&x)[16]) {
        const float4 *p4 = reinterpret_cast<const float4 *>(st + 32 * t + 8 * lh);
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const float4 f4 = p4[4 * (g >> 1) + (g & 1)];
            x[4 * g] = f4.x;
            x[4 * g + 1] = f4.y;
            x[4 * g + 2] = f4.z;
            x[4 * g + 3] = f4.w;
        }
    };
    // score-type product of this wave's 32 keys with the 32 rows of tile t of
    // `rt` (Q for S, dO for dP), accumulated onto `init`; row operands read
    // two products ahead.
    auto score = [&](const char *rt, int t, const frag (&f)[KS], const f32x16 &init) -> f32x16 {
        f32x16 acc = init;
        const int row = 32 * t + O::pi(li);
        constexpr int PF = 2, NSL = PF + 1;
        frag ra[NSL];
        auto ld = [&](int ks) {
            if (ks < KS) ra[ks % NSL] = Tl::frag_row(rt, row, ks * O::KW + lh * O::KL);
        };
#pragma unroll
        for (int g = 0; g < PF; ++g) ld(g);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            ld(ks + PF);
            acc = O::mma(ra[ks % NSL], f[ks], acc);
            __builtin_amdgcn_sched_barrier(0);
        }
        return acc;
    };

    // The queue walk, instantiated once per role: the two roles run separate
    // loops (so that the compiler keeps each role's accumulators in place)
    // that pass the same barriers in the same order.
    auto walk = [&](auto role_tag) {
        constexpr int ROLE = decltype(role_tag)::value;
        // First item: its K/V into buffer 1, its first stage into buffer 0.
        int e = e0;
        int4 cur = item(e);
        issue_kv(1, cur.x);
        if (cur.z > cur.y) issue_stage(0, rows[cur.y]);
        wait_vmcnt<0>();
        barrier_lds();
        frag kv[KS];  // K fragments (role 0) or V fragments (role 1)
        load_frags(1, kv);
        int sb = 0;  // buffer holding the current item's first stage

        for (;;) {
            const int nstage = cur.z - cur.y;
            const bool more = e + 1 < e1;
            const int4 nxt = more ? item(e + 1) : make_int4(0, 0, 0, 0);
            scalar_ready(nxt);  // see dkdv_queue_kernel
            f32x16 acc[DT];     // dV (role 0) or dK (role 1), transposed: lane = key
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
            if (nstage == 0 && more) issue_kv(sb, nxt.x);
            const int ntile = 4 * nstage;
            [[maybe_unused]] f32x16 dp = zero16();  // role 1: dP of the tile it finishes next
            // role 1: dS and dK of tile t of stage j (in buffer b), P from
            // LDS. The tile index is a compile-time constant here and in the
            // stage body below (its four tiles are unrolled), so that the
            // LDS addresses of a stage are one base plus immediate offsets.
            auto finish = [&](int j, int b, auto t_tag) {
                constexpr int t = decltype(t_tag)::value;
                const char *qt = buffer(b);
                frag pr[VPK];
#pragma unroll
                for (int kk = 0; kk < VPK; ++kk) pr[kk] = s_p[t & 1][pair][kk][lane];
                // the dK product's transposed Q operands, read before the dS
                // arithmetic that waits for P
                frag tq[VPK * DT];
#pragma unroll
                for (int g = 0; g < VPK * DT; ++g)
                    tq[g] = Tl::frag_tr(qt, 32 * t + (g / DT) * O::KW, 32 * (g % DT), lane);
                __builtin_amdgcn_sched_barrier(0);
                f32x16 dsv;
#pragma unroll
                for (int v = 0; v < 16; ++v)
                    dsv[v] = static_cast<float>(pr[v / O::KL][v % O::KL]) * dp[v];  // dp holds dP - D
                frag bd[VPK];
#pragma unroll
                for (int kk = 0; kk < VPK; ++kk) bd[kk] = O::pack(dsv, kk * O::KL);
                if constexpr (DS) {
                    const int blk = as_const(a.bsc_block)[cur.y + j];
                    asm volatile("" ::"s"(blk));
                    T *dsr = static_cast<T *>(a.ds) +
                             ((static_cast<size_t>(bh) * a.nnzb + blk) * BLK + 32 * pair + li) * BLK;
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk)
                        *reinterpret_cast<frag *>(dsr + 32 * t + 16 * kk + 8 * lh) = bd[kk];
                }
#pragma unroll
                for (int g = 0; g < VPK * DT; ++g) acc[g % DT] = O::mma(tq[g], bd[g / DT], acc[g % DT]);
            };
            using T0 = std::integral_constant<int, 0>;
            using T1 = std::integral_constant<int, 1>;
            using T2 = std::integral_constant<int, 2>;
            using T3 = std::integral_constant<int, 3>;
            if (ntile > 0) {
                wait_vmcnt<0>();
                barrier_lds();  // first stage visible; every wave done with the previous item
            }
            for (int j = 0; j < nstage; ++j) {
                const int b = (sb + j) & 1;
                const char *qt = buffer(b), *ot = buffer(b) + TILE;
                auto tile = [&](auto t_tag) {
                    constexpr int t = decltype(t_tag)::value;
                    if constexpr (ROLE == 0) {
                        float ls[16];
                        stats(s_lse[b], t, ls);
                        f32x16 sv = score(qt, t, kv, zero16());
                        // the dV product's transposed dO operands, read before
                        // the softmax that waits for the scores
                        frag to[VPK * DT];
#pragma unroll
                        for (int g = 0; g < VPK * DT; ++g)
                            to[g] = Tl::frag_tr(ot, 32 * t + (g / DT) * O::KW, 32 * (g % DT), lane);
                        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                        for (int v = 0; v < 16; ++v) sv[v] = exp2_fast(fmaf(sv[v], a.c, -ls[v]));
                        frag bp[VPK];
#pragma unroll
                        for (int kk = 0; kk < VPK; ++kk) {
                            bp[kk] = O::pack(sv, kk * O::KL);
                            s_p[t & 1][pair][kk][lane] = bp[kk];
                        }
#pragma unroll
                        for (int g = 0; g < VPK * DT; ++g) acc[g % DT] = O::mma(to[g], bp[g / DT], acc[g % DT]);
                    } else {
                        if constexpr (t > 0) finish(j, b, std::integral_constant<int, t - 1>{});
                        else if (j > 0) finish(j - 1, b ^ 1, T3{});
                        // dP - D in one accumulation: the products start from the
                        // tile's -D (stored negated by the dQ pass or prep)
                        float dl[16];
                        stats(s_dlt[b], t, dl);
                        f32x16 init;
#pragma unroll
                        for (int v = 0; v < 16; ++v) init[v] = dl[v];
                        dp = score(ot, t, kv, init);
                    }
                    if constexpr (t == 3) {
                        if (j + 1 < nstage) wait_vmcnt<0>();  // this wave's copies of stage j + 1
                    }
                    barrier_lds();  // P of tile t visible; stage j + 1 visible after the last tile of stage j
                    if constexpr (ROLE == 0 && t == 0) {
                        // every wave is done with stage j - 1: refill its buffer
                        if (j + 1 < nstage) issue_stage(b ^ 1, rows[cur.y + j + 1]);
                        else if (more) issue_kv(b ^ 1, nxt.x);
                    }
                };
                tile(T0{});
                tile(T1{});
                tile(T2{});
                tile(T3{});
            }
            if constexpr (ROLE == 1) {
                if (ntile > 0) finish(nstage - 1, (sb + nstage - 1) & 1, T3{});
            }
            const int F = (sb + nstage) & 1;  // free buffer; holds the next K/V when there is a next item
            if (more) {
                wait_vmcnt<0>();
                barrier_lds();  // next K/V visible; every wave done with the last stage
                if (nxt.z > nxt.y) issue_stage(F ^ 1, rows[nxt.y]);
                load_frags(F, kv);
            }
            // Outputs: role 0 writes dV, role 1 dK (scaled), each staged
            // through this wave's own 32 rows of the K (role 0) or V (role 1)
            // tile in buffer F, which it has just read into registers.
            const int J = cur.x, slot = cur.w;
            const float mul = ROLE ? a.scale : 1.f;
            if (slot < 0) {
                char *sk = buffer(F) + ROLE * TILE + 32 * pair * D * 2;
                __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
                T *dst = static_cast<T *>(ROLE ? a.dk : a.dv) + base + static_cast<size_t>(J * BLK + 32 * pair) * D;
                store_tile_lds<D, DT>(sk, dst, acc, mul, lane);
            } else {
                const int ln = opaque(lane);
                const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * pair + (ln & 31);
                store_rows<DT>((ROLE ? a.part_dk : a.part_dv) + prow * D, acc, mul, ln >> 5);
            }
            if (!more) break;
            ++e;
            cur = nxt;
            sb = F ^ 1;
        }
    };
    if (role == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});
}

// Column-first dK/dV at head_dim 256 with two waves per SIMD (bf16/fp16):
// 512 threads, the 128 keys of one column item, the roles of
// dkdv_pair_kernel (the two waves that own the same 32 keys split each
// 32-query tile):
//   role 0 (waves 0-3):  K rows in registers; S = Q_t K^T, P = 2^(S*c - lse2),
//                        P packed into LDS, dV^T += dO_t^T P;
//   role 1 (waves 4-7):  V rows in registers; dP - delta = dO_t V^T
//                        accumulated onto -delta; one tile later, with P from
//                        LDS, dS = P (dP - delta) and dK^T += Q_t^T dS.
// Each wave holds one 32 x 256 operand and one 256-wide accumulator (one
// wave holding both of each needs ~400 registers: one wave per SIMD, as the
// fp32 dkdv_kernel runs). Operand addresses
// are formed per tile and the row operands of the score products share
// eight chunk offsets, which keeps both roles within 256 registers.
// 32-query stages of Q and dO in a ring of four buffers filled by LDS-DMA
// (Q by the role-0 waves; dO, lse2 and delta by the role-1 waves, so that
// the two waves of a SIMD issue equal shares): a buffer is refilled after
// the barrier that ends role 1's use of it, three stages ahead, so copies
// have two tiles of lead. One barrier per tile. Operand rings two products
// ahead. (dS here is formed from P as rounded for the dV product.)
// DS: role 1 also stores each tile's dS^T (as rounded for the dK product)
// for the dQ pass that reads it, in dkdv_stage's layout.
// C4 (1x8x8192x256, random 10 %): dK/dV 168 -> 136 us against the one-wave
// form it replaced, storing dS 213 -> 153 us.
template <typename T, int D, bool DS = false>
__global__ void __launch_bounds__(NT2, 1) dkdv_wide_pair_kernel(DkdvArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, D>;
    using frag = typename O::frag;
    static_assert(sizeof(T) == 2 && D == 256, "16-bit operands, head_dim 256");
    constexpr int SB = 32;                    // query rows per stage: one tile
    constexpr int NSUB = BLK / SB;            // stages per block row
    constexpr int NBUF = 4;                   // stage buffers in the ring
    constexpr int TILE = SB * D * sizeof(T);  // one staged Q or dO tile
    constexpr int KS = D / O::KW;             // k-steps over head_dim
    constexpr int DT = D / 32;                // 32-column accumulator tiles
    constexpr int VPK = 32 / O::KW;           // k-steps per 32-query tile
    using AT = AsyncTile<D, SB, NT>;          // one tile's copies, issued by the 256 threads of a role
    static_assert(KS == 16, "eight chunk offsets per row");
    __shared__ __attribute__((aligned(16))) char smem[NBUF * 2 * TILE];
    __shared__ __attribute__((aligned(16))) float s_lse[NBUF][SB], s_dlt[NBUF][SB];
    __shared__ __attribute__((aligned(16))) frag s_p[2][4][VPK][64];  // [tile parity][pair][k-step][lane]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & 3, role = w >> 2;
    const int li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int J = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *dO = static_cast<const T *>(a.dout) + base;
    const float *LSE = a.lse2 + static_cast<size_t>(bh) * a.S;
    const float *DLT = a.delta + static_cast<size_t>(bh) * a.S;
    const int kr = J * BLK + 32 * pair + li;  // this lane's key row
    const int nstage = (p1 - p0) * NSUB;
    const auto tp = AT::plan(tid & (NT - 1));
    const const_i32 *rows = as_const(a.row_idx);
    auto buffer = [&](int k) { return smem + (k & (NBUF - 1)) * 2 * TILE; };
    // Stage k: its Q rows (role-0 waves), its dO rows and the lse2 and delta
    // of its 32 queries (role-1 waves; 16 values per wave).
    auto issue_stage = [&](int k) {
        const size_t r0 = static_cast<size_t>(rows[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
        if (role == 0) {
            AT::issue(tp, buffer(k), Q + r0 * D);
        } else {
            AT::issue(tp, buffer(k) + TILE, dO + r0 * D);
            // waves 4, 5: lse2 halves; waves 6, 7: delta halves
            const int h16 = 16 * (w & 1);
            float *dst = (w < 6 ? &s_lse[k & (NBUF - 1)][0] : &s_dlt[k & (NBUF - 1)][0]) + h16;
            if (lane < 16) dma4((w < 6 ? LSE : DLT) + r0 + h16 + lane, dst);
        }
    };

    auto walk = [&](auto role_tag) {
        constexpr int ROLE = decltype(role_tag)::value;
        constexpr int L = AT::LOADS + ROLE;  // loads per stage of a wave
        const T *KV = static_cast<const T *>(ROLE ? a.v : a.k) + base;
        frag f[KS];  // K (role 0) or V (role 1) rows of this lane's key
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) f[ks] = gfrag(KV + static_cast<size_t>(kr) * D + ks * O::KW + lh * O::KL);
        f32x16 acc[DT];  // dV (role 0) or dK (role 1), transposed: lane = key
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
        for (int k = 0; k < NBUF - 1 && k < nstage; ++k) issue_stage(k);
        if (nstage >= 3) wait_vmcnt<2 * L>();
        else if (nstage == 2) wait_vmcnt<L>();
        else wait_vmcnt<0>();
        barrier_lds();  // stage 0 visible

        // score-type product of this wave's 32 keys with the tile of `rt`,
        // onto `x`; row operands one product ahead
        auto score = [&](const char *rt, f32x16 x) -> f32x16 {
            const int ln = opaque(lane);
            const int row = O::pi(ln & 31), lq = ln >> 5;
            constexpr int PF = 2, NS = PF + 1;
            frag ra[NS];
            auto ld = [&](int ks) {
                if (ks < KS)
                    ra[ks % NS] = *reinterpret_cast<const frag *>(
                        rt + Tl::off(row, ((ks & 7) * O::KW + lq * O::KL) >> 3) + (ks >> 3) * 256);
            };
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                ld(ks + PF);
                x = O::mma(ra[ks % NS], f[ks], x);
                __builtin_amdgcn_sched_barrier(0);
            }
            return x;
        };
        // acc += (tile of `tt`)^T B over the tile's 32 rows; transposed
        // operands one product ahead. The reads are Tile16::frag_tr's: a
        // lane reads rows r0 and r0 + 4 at chunk 4 dt + cx of column group
        // dt. Groups dt and dt + 4 are 16 chunks (256 bytes) apart, which the
        // swizzle (low four chunk bits, row % 16) preserves, and the two
        // k-steps 16 rows apart, which it ignores: four offsets per read row
        // serve all sixteen operands.
        auto accumulate = [&](const char *tt, const frag (&bb)[VPK]) {
            const int ln = opaque(lane);
            const int cx = 2 * ((ln >> 4) & 1) + ((ln & 3) >> 1), sub = 8 * (ln & 1);
            const int r0 = 8 * (ln >> 5) + ((ln & 15) >> 2);
            uint32_t o0[4], o1[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                o0[d] = Tl::off(r0, 4 * d + cx) + sub;
                o1[d] = Tl::off(r0 + 4, 4 * d + cx) + sub;
            }
            auto rd = [&](int g) -> frag {
                const int dt = g % DT;
                const uint32_t add = (dt >> 2) * 256 + (g / DT) * O::KW * (D * 2);
                s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tt + o0[dt & 3] + add));
                s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4 *)(tt + o1[dt & 3] + add));
                s16x8 both = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                return __builtin_bit_cast(frag, both);
            };
            static_assert(DT == 8, "two groups of four column groups");
            constexpr int PF = 2, NS = PF + 1, NG = VPK * DT;
            frag ta[NS];
            auto ld = [&](int g) {
                if (g < NG) ta[g % NS] = rd(g);
            };
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                ld(g + PF);
                acc[g % DT] = O::mma(ta[g % NS], bb[g / DT], acc[g % DT]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        // the value v of a lane belongs to query pi(8(v/4) + 4(lane/32) + v%4)
        auto qidx = [&](int v) { return O::pi(8 * (v >> 2) + 4 * lh + (v & 3)); };

        [[maybe_unused]] f32x16 dp;  // role 1: dP - delta of the tile it finishes next
        for (int t = 0; t <= nstage; ++t) {
            const int b = t & (NBUF - 1);
            if constexpr (ROLE == 0) {
                if (t < nstage) {
                    const char *qt = buffer(t), *ot = qt + TILE;
                    f32x16 sv = score(qt, zero16());
#pragma unroll
                    for (int v = 0; v < 16; ++v) sv[v] = exp2_fast(fmaf(sv[v], a.c, -s_lse[b][qidx(v)]));
                    frag bp[VPK];
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk) {
                        bp[kk] = O::pack(sv, kk * O::KL);
                        s_p[t & 1][pair][kk][lane] = bp[kk];
                    }
                    accumulate(ot, bp);
                }
            } else {
                if (t > 0) {
                    // finish tile t - 1: dS from its P, dK^T += Q^T dS
                    frag pr[VPK];
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk) pr[kk] = s_p[(t - 1) & 1][pair][kk][lane];
#pragma unroll
                    for (int v = 0; v < 16; ++v) dp[v] = static_cast<float>(pr[v / O::KL][v % O::KL]) * dp[v];
                    frag bd[VPK];
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk) bd[kk] = O::pack(dp, kk * O::KL);
                    if constexpr (DS) {
                        // dS^T of tile t - 1: the lane's key row of its block, 32 queries from the tile's first
                        const int k = t - 1;
                        const int blk = as_const(a.bsc_block)[p0 + k / NSUB];
                        T *dsr = static_cast<T *>(a.ds) +
                                 ((static_cast<size_t>(bh) * a.nnzb + blk) * BLK + 32 * pair + li) * BLK + (k % NSUB) * SB;
#pragma unroll
                        for (int kk = 0; kk < VPK; ++kk) *reinterpret_cast<frag *>(dsr + 16 * kk + 8 * lh) = bd[kk];
                    }
                    accumulate(buffer(t - 1), bd);
                }
                if (t < nstage) {
                    f32x16 init;
#pragma unroll
                    for (int v = 0; v < 16; ++v) init[v] = s_dlt[b][qidx(v)];
                    dp = score(buffer(t) + TILE, init);
                }
            }
            // this wave's loads of stage t + 1 (stage t + 2 may stay in flight)
            if (t + 2 < nstage) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            barrier_lds();  // P of tile t and stage t + 1 visible; every wave done with stage t - 1
            if (t + NBUF - 1 < nstage) issue_stage(t + NBUF - 1);  // into the buffer of stage t - 1
        }
        // Outputs: role 0 dV, role 1 dK (scaled); each wave stages its 32 x 256
        // tile through its own 16 KB of the (now unused) stage buffers.
        const float mul = ROLE ? a.scale : 1.f;
        if (slot < 0) {
            T *dst = static_cast<T *>(ROLE ? a.dk : a.dv) + base + static_cast<size_t>(J * BLK + 32 * pair) * D;
            store_tile_lds<D, DT>(smem + w * (32 * D * 2), dst, acc, mul, lane);
        } else {
            const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * pair + li;
            store_rows<DT>((ROLE ? a.part_dk : a.part_dv) + prow * D, acc, mul, lh);
        }
    };
    if (role == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});
}

// Forward with two waves per SIMD that split the work of each 32-key tile by
// role (bf16/fp16): 512 threads, the 128 query rows of one row item; the two
// waves that own the same 32 query rows:
//   role 0 (waves 0-3):  S^T = K_t Q^T (lane = query), the running row
//                        maximum and sum with the reference raised lazily as
//                        in fwd_kernel, P packed to LDS in the form the P V
//                        product reads, and the factor that rescales O when
//                        the reference rises (1 otherwise);
//   role 1 (waves 4-7):  O^T = O^T * factor + V_t^T P for the tile role 0
//                        finished in the previous interval.
// Role 0 has all the softmax work and role 1 none, so the two waves of a
// SIMD cover each other's vector work, LDS waits and barriers, and at
// head_dim 256 each holds one of the two register sets (Q, or the 256-wide
// accumulator) that the one-wave forward holds together. One barrier per
// tile; 32-key stages of K and V (one tile) in a ring of four buffers filled
// by LDS-DMA (K by the role-0 waves, V by the role-1 waves), a buffer
// refilled after the barrier that ends role 1's use of it, three stages
// ahead. P and the factors go through double buffers.
template <typename T, int D>
__global__ void __launch_bounds__(NT2, 1) fwd_pair_kernel(FwdArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, D>;
    using frag = typename O::frag;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int SB = 32;                    // keys per stage: one tile
    constexpr int NSUB = BLK / SB;            // stages per key block
    constexpr int NBUF = 4;                   // stage buffers in the ring
    constexpr int TILE = SB * D * sizeof(T);  // one staged K or V tile
    using AT = AsyncTile<D, SB, NT>;          // one tile's copies, issued by the 256 threads of a role
    constexpr int KS = D / O::KW;
    constexpr int DT = D / 32;
    constexpr int VPK = 32 / O::KW;
    __shared__ __attribute__((aligned(16))) char smem[NBUF * 2 * TILE];
    __shared__ __attribute__((aligned(16))) frag s_p[2][4][VPK][64];  // [tile parity][pair][k-step][lane]
    __shared__ float s_fac[2][4][32];                                 // [tile parity][pair][query]
    __shared__ float s_inv[4][32];                                    // [pair][query]: 1 / row sum

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & 3, role = w >> 2;
    const int li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *Q = static_cast<const T *>(a.q) + base;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const int qr = I * BLK + 32 * pair + li;  // this lane's query row
    const int nstage = (p1 - p0) * NSUB;
    const const_i32 *cols = as_const(a.col_idx);
    const auto tp = AT::plan(tid & (NT - 1));
    auto buffer = [&](int k) { return smem + (k & (NBUF - 1)) * 2 * TILE; };
    // stage k: its K rows (role-0 waves) and V rows (role-1 waves)
    auto issue_stage = [&](int k) {
        const size_t r0 = static_cast<size_t>(cols[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
        if (role == 0) AT::issue(tp, buffer(k), K + r0 * D);
        else AT::issue(tp, buffer(k) + TILE, V + r0 * D);
    };

    auto walk = [&](auto role_tag) {
        constexpr int ROLE = decltype(role_tag)::value;
        constexpr int L = AT::LOADS;  // loads per stage of every wave
        // role 0: Q fragments; running statistics in base-2 units (m2 the
        // reference the exponentials are taken against, mx2 the exact max)
        [[maybe_unused]] frag qf[ROLE == 0 ? KS : 1];
        [[maybe_unused]] float m2 = -INFINITY, mx2 = -INFINITY, lsum = 0.f;
        // role 1: the output accumulator (transposed: lane = query)
        [[maybe_unused]] f32x16 acc[ROLE == 1 ? DT : 1];
        if constexpr (ROLE == 0) {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qf[ks] = gfrag(Q + static_cast<size_t>(qr) * D + ks * O::KW + lh * O::KL);
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
        }
        for (int k = 0; k < NBUF - 1 && k < nstage; ++k) issue_stage(k);
        if (nstage >= 3) wait_vmcnt<2 * L>();
        else if (nstage == 2) wait_vmcnt<L>();
        else wait_vmcnt<0>();
        barrier_lds();  // stage 0 visible
        // role 1: rescale and accumulate the tile of stage k
        auto finish = [&](int par, int k) {
            constexpr int t = 0;
            const char *vt = buffer(k) + TILE;
            frag pf[VPK];
#pragma unroll
            for (int kk = 0; kk < VPK; ++kk) pf[kk] = s_p[par][pair][kk][lane];
            const float fac = s_fac[par][pair][li];
            if (__any(fac != 1.f)) {  // rare: the reference of some row rose
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[dt][v] *= fac;
            }
            constexpr int PF = 2, NS = PF + 1, NG = VPK * DT;
            frag vb[NS];
            auto ld = [&](int g) {
                if (g < NG) vb[g % NS] = Tl::frag_tr(vt, 32 * t + (g / DT) * O::KW, 32 * (g % DT), lane);
            };
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                ld(g + PF);
                acc[g % DT] = O::mma(vb[g % NS], pf[g / DT], acc[g % DT]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int k = 0; k <= nstage; ++k) {
            const int par = k & 1;
            if constexpr (ROLE == 0) {
                if (k < nstage) {
                    const char *kt = buffer(k);
                    f32x16 s = zero16();
                    const int row = O::pi(li);
                    constexpr int PF = 2, NS = PF + 1;
                    frag ka[NS];
                    auto ld = [&](int ks) {
                        if (ks < KS) ka[ks % NS] = Tl::frag_row(kt, row, ks * O::KW + lh * O::KL);
                    };
#pragma unroll
                    for (int g = 0; g < PF; ++g) ld(g);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        ld(ks + PF);
                        s = O::mma(ka[ks % NS], qf[ks], s);
                        __builtin_amdgcn_sched_barrier(0);
                    }
                    float mx = -INFINITY;
#pragma unroll
                    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, s[v]);
                    mx = pair_max(mx) * a.c;
                    mx2 = fmaxf(mx2, mx);
                    float fac = 1.f;
                    if (k == 0) {
                        m2 = mx;  // nothing accumulated yet
                    } else if (mx > m2 + RESCALE_LOG2) {
                        fac = exp2_fast(m2 - mx);
                        lsum *= fac;
                        m2 = mx;
                    }
                    if (lh == 0) s_fac[par][pair][li] = fac;
                    float rs = 0.f;
#pragma unroll
                    for (int v = 0; v < 16; ++v) s[v] = exp2_fast(fmaf(s[v], a.c, -m2));
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk) {
                        const frag pf = O::pack(s, kk * O::KL);
                        rs = rowsum_acc(pf, rs);  // the row sum of the rounded P the product uses
                        s_p[par][pair][kk][lane] = pf;
                    }
                    lsum += pair_sum(rs);
                }
            } else {
                if (k > 0) finish(par ^ 1, k - 1);
            }
            // this wave's loads of stage k + 1 (stage k + 2 may stay in flight)
            if (k + 2 < nstage) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            barrier_lds();  // P of tile k and stage k + 1 visible; every wave done with stage k - 1
            if (k + NBUF - 1 < nstage) issue_stage(k + NBUF - 1);  // into the buffer of stage k - 1
        }
        if constexpr (ROLE == 0) {
            if (lh == 0) s_inv[pair][li] = slot < 0 ? (lsum > 0.f ? 1.f / lsum : 0.f) : 1.f;
        }
        barrier_lds();  // the row sums visible
        const size_t srow = static_cast<size_t>(bh) * a.S + qr;
        if constexpr (ROLE == 1) {
            const float inv = s_inv[pair][li];
            if (slot < 0) {
                char *scratch = smem + pair * (32 * D * 2);
                store_tile_lds<D, DT>(scratch, static_cast<T *>(a.o) + base + static_cast<size_t>(I * BLK + 32 * pair) * D,
                                      acc, inv, lane);
            } else {
                const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * pair + li;
                store_rows<DT>(a.part_o + prow * D, acc, 1.f, lh);
            }
        } else if (lh == 0) {
            if (slot < 0) {
                a.row_max[srow] = lsum > 0.f ? mx2 / LOG2E : -INFINITY;
                a.row_denom[srow] = lsum > 0.f ? lsum * exp2_fast(m2 - mx2) : 0.f;
            } else {
                const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * pair + li;
                a.part_m2[prow] = m2;
                a.part_l[prow] = lsum;
                a.part_mx[prow] = mx2;
            }
        }
    };
    if (role == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});
}

// Row-first dQ split by role over two waves per SIMD (bf16/fp16), the same
// arrangement as fwd_pair_kernel: 512 threads, the 128 query rows of one row
// item; the two waves that own the same 32 query rows:
//   role 0 (waves 0-3):  Q and dO rows in registers; the row terms (delta,
//                        lse2) as dq_kernel forms them; per 32-key tile
//                        S^T = K_t Q^T and dP^T = V_t dO^T (lane = query),
//                        P = 2^(S*c - lse2), dS = P (dP - delta), dS packed
//                        to LDS in the form the dQ product reads;
//   role 1 (waves 4-7):  dQ^T += K_t^T dS for the tile role 0 finished in
//                        the previous interval (the 256-wide accumulator).
// 32-key stages of K and V (one tile) in a ring of four buffers filled by
// LDS-DMA (K by the role-0 waves, V by the role-1 waves), a buffer refilled
// after the barrier that ends role 1's use of it, three stages ahead (two
// tiles of lead; with 64-key stages double-buffered there was one, and dQ
// took 105.4 against 104.6 us on C4); one barrier per tile; dS goes through
// a double buffer.
template <typename T, int D>
__global__ void __launch_bounds__(NT2, 1) dq_pair_kernel(DqArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, D>;
    using frag = typename O::frag;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int SB = 32;                    // keys per stage: one tile
    constexpr int NSUB = BLK / SB;            // stages per key block
    constexpr int NBUF = 4;                   // stage buffers in the ring
    constexpr int TILE = SB * D * sizeof(T);  // one staged K or V tile
    using AT = AsyncTile<D, SB, NT>;          // one tile's copies, issued by the 256 threads of a role
    constexpr int KS = D / O::KW;
    constexpr int DT = D / 32;
    constexpr int VPK = 32 / O::KW;
    __shared__ __attribute__((aligned(16))) char smem[NBUF * 2 * TILE];
    __shared__ __attribute__((aligned(16))) frag s_ds[2][4][VPK][64];  // [tile parity][pair][k-step][lane]

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int pair = w & 3, role = w >> 2;
    const int li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *V = static_cast<const T *>(a.v) + base;
    const int qr = I * BLK + 32 * pair + li;  // this lane's query row
    const int nstage = (p1 - p0) * NSUB;
    const const_i32 *cols = as_const(a.col_idx);
    const auto tp = AT::plan(tid & (NT - 1));
    auto buffer = [&](int k) { return smem + (k & (NBUF - 1)) * 2 * TILE; };
    // stage k: its K rows (role-0 waves) and V rows (role-1 waves)
    auto issue_stage = [&](int k) {
        const size_t r0 = static_cast<size_t>(cols[p0 + k / NSUB]) * BLK + (k % NSUB) * SB;
        if (role == 0) AT::issue(tp, buffer(k), K + r0 * D);
        else AT::issue(tp, buffer(k) + TILE, V + r0 * D);
    };

    auto walk = [&](auto role_tag) {
        constexpr int ROLE = decltype(role_tag)::value;
        constexpr int L = AT::LOADS;  // loads per stage of every wave
        [[maybe_unused]] frag qf[ROLE == 0 ? KS : 1], df[ROLE == 0 ? KS : 1];
        [[maybe_unused]] float dlt = 0.f, lse = 0.f;
        [[maybe_unused]] f32x16 acc[ROLE == 1 ? DT : 1];  // dQ^T, lane = query
        if constexpr (ROLE == 0) {
            const size_t srow = static_cast<size_t>(bh) * a.S + qr;
            const T *Q = static_cast<const T *>(a.q) + base, *dO = static_cast<const T *>(a.dout) + base;
            const T *Ob = static_cast<const T *>(a.o) + base;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const size_t off = static_cast<size_t>(qr) * D + ks * O::KW + lh * O::KL;
                qf[ks] = gfrag(Q + off);
                df[ks] = gfrag(dO + off);
                dlt = frag_dot(gfrag(Ob + off), df[ks], dlt);
            }
            dlt = pair_sum(dlt);
            const float rden = a.row_denom[srow];
            lse = rden > 0.f ? fmaf(a.row_max[srow], LOG2E, log2f(rden)) : INFINITY;
            if (lh == 0 && (slot < 0 || p0 == as_const(a.row_ptr)[I])) {
                a.delta[srow] = -dlt;  // stored negated (see dkdv_pair_kernel)
                a.lse2[srow] = lse;
            }
        } else {
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
        }
        for (int k = 0; k < NBUF - 1 && k < nstage; ++k) issue_stage(k);
        if (nstage >= 3) wait_vmcnt<2 * L>();
        else if (nstage == 2) wait_vmcnt<L>();
        else wait_vmcnt<0>();
        barrier_lds();  // stage 0 visible
        // role 1: dQ^T += K^T dS for the tile of stage k
        auto finish = [&](int par, int k) {
            constexpr int t = 0;
            const char *kt = buffer(k);
            frag bd[VPK];
#pragma unroll
            for (int kk = 0; kk < VPK; ++kk) bd[kk] = s_ds[par][pair][kk][lane];
            constexpr int PF = 2, NS = PF + 1, NG = VPK * DT;
            frag kb[NS];
            auto ld = [&](int g) {
                if (g < NG) kb[g % NS] = Tl::frag_tr(kt, 32 * t + (g / DT) * O::KW, 32 * (g % DT), lane);
            };
#pragma unroll
            for (int g = 0; g < PF; ++g) ld(g);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                ld(g + PF);
                acc[g % DT] = O::mma(kb[g % NS], bd[g / DT], acc[g % DT]);
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        for (int k = 0; k <= nstage; ++k) {
            const int par = k & 1;
            if constexpr (ROLE == 0) {
                if (k < nstage) {
                    const char *kt = buffer(k), *vt = kt + TILE;
                    f32x16 sc = zero16(), dp;  // dp: dP - delta, the products starting from -delta
#pragma unroll
                    for (int v = 0; v < 16; ++v) dp[v] = -dlt;
                    const int row = O::pi(li);
                    constexpr int PF = 2, NS = PF + 1;
                    frag ka[NS], va[NS];
                    auto ld = [&](int ks) {
                        if (ks < KS) {
                            ka[ks % NS] = Tl::frag_row(kt, row, ks * O::KW + lh * O::KL);
                            va[ks % NS] = Tl::frag_row(vt, row, ks * O::KW + lh * O::KL);
                        }
                    };
#pragma unroll
                    for (int g = 0; g < PF; ++g) ld(g);
                    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        ld(ks + PF);
                        sc = O::mma(ka[ks % NS], qf[ks], sc);
                        dp = O::mma(va[ks % NS], df[ks], dp);
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const float p = exp2_fast(fmaf(sc[v], a.c, -lse));
                        sc[v] = p * dp[v];
                    }
#pragma unroll
                    for (int kk = 0; kk < VPK; ++kk) s_ds[par][pair][kk][lane] = O::pack(sc, kk * O::KL);
                }
            } else {
                if (k > 0) finish(par ^ 1, k - 1);
            }
            // this wave's loads of stage k + 1 (stage k + 2 may stay in flight)
            if (k + 2 < nstage) wait_vmcnt<L>();
            else wait_vmcnt<0>();
            barrier_lds();  // dS of tile k and stage k + 1 visible; every wave done with stage k - 1
            if (k + NBUF - 1 < nstage) issue_stage(k + NBUF - 1);  // into the buffer of stage k - 1
        }
        if constexpr (ROLE == 1) {
            if (slot < 0) {
                char *scratch = smem + pair * (32 * D * 2);
                store_tile_lds<D, DT>(scratch, static_cast<T *>(a.dq) + base + static_cast<size_t>(I * BLK + 32 * pair) * D,
                                      acc, a.scale, lane);
            } else {
                const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * pair + li;
                store_rows<DT>(a.part + prow * D, acc, a.scale, lh);
            }
        }
    };
    if (role == 0) walk(std::integral_constant<int, 0>{});
    else walk(std::integral_constant<int, 1>{});
}

// Row terms of the backward for the schedule that runs dK/dV before dQ (the
// dS-storing backward): delta = rowsum(dO * O) over the returned O and
// lse2 = row_max * log2(e) + log2(row_denom) (+inf for an empty row), the
// same quantities the dQ pass forms in its prologue. D/8 lanes per row, one
// 16-byte chunk of O and dO each.
struct PrepArgs {
    const void *o, *dout;
    const float *row_max, *row_denom;
    float *delta, *lse2;
    int64_t rows;
};

template <typename T, int D>
__global__ void __launch_bounds__(NT) prep_kernel(PrepArgs a) {
    constexpr int CH = D / 8;    // lanes per row
    constexpr int RB = NT / CH;  // rows per pass of the workgroup
    constexpr int RPT = 4;       // passes: rows per thread, all loads issued first
    const int tid = threadIdx.x, c = tid % CH;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * RB * RPT + tid / CH;
    const T *O = static_cast<const T *>(a.o);
    const T *dO = static_cast<const T *>(a.dout);
    // Rows past the end load the last row (no branch between the loads) and
    // store nothing. The row statistics are loaded with O and dO, so that
    // the only wait is for this one round of loads.
    typename Op<T>::frag x[RPT], y[RPT];
    float rmax[RPT], rden[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t row = row0 + i * RB < a.rows ? row0 + i * RB : a.rows - 1;
        x[i] = gfrag(O + static_cast<size_t>(row) * D + c * 8);
        y[i] = gfrag(dO + static_cast<size_t>(row) * D + c * 8);
        rmax[i] = a.row_max[row];
        rden[i] = a.row_denom[row];
    }
    float acc[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) acc[i] = frag_dot(x[i], y[i], 0.f);
#pragma unroll
    for (int m = CH / 2; m >= 1; m >>= 1)
#pragma unroll
        for (int i = 0; i < RPT; ++i) acc[i] += __shfl_xor(acc[i], m, CH);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int64_t row = row0 + i * RB;
        if (row < a.rows && c == 0) {
            a.delta[row] = -acc[i];  // stored negated, as the dQ pass stores it
            a.lse2[row] = rden[i] > 0.f ? fmaf(rmax[i], LOG2E, log2f(rden[i])) : INFINITY;
        }
    }
}

struct DqDsArgs {
    const void *k, *ds;  // ds: dS^T blocks [BH][nnzb][128 keys][128 queries], by BSR position
    void *dq;
    const int4 *items;
    const int32_t *col_idx;
    float *part;
    int BH, S, nnzb;
    float scale;
};

// dQ from the stored dS (the dS-storing backward, where the dK/dV pass wrote
// dS): for each stored block J of the row (BSR position p), in SB-key
// sub-blocks of K_J and of the block's dS^T, both staged in LDS by LDS-DMA
// and read with transposing reads, dQ^T += K_J^T dS_IJ^T; dQ = scale * dQ.
// No scores are recomputed. Items, outputs and partial slots are those of
// the dQ pass that recomputes dS.
template <typename T, int D, int SB, int MINW>
__global__ void __launch_bounds__(NT, MINW) dq_ds_kernel(DqDsArgs a) {
    using O = Op<T>;
    using Tk = Tile<T, D>;
    using Ts = Tile<T, BLK>;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int KT = SB * D * 2, ST = SB * BLK * 2, BUF = KT + ST;
    constexpr int NSUB = BLK / SB;
    constexpr int DT = D / 32;
    __shared__ __attribute__((aligned(16))) char smem[2 * BUF];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, lh = lane >> 5;
    const int item = blockIdx.x / a.BH, bh = blockIdx.x % a.BH;
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const T *K = static_cast<const T *>(a.k) + base;
    const T *dS = static_cast<const T *>(a.ds) + static_cast<size_t>(bh) * a.nnzb * BLK * BLK;
    const auto tk = AsyncTile<D, SB>::plan(tid);
    const auto ts = AsyncTile<BLK, SB>::plan(tid);
    const const_i32 *cols = as_const(a.col_idx);
    // Sub-block k of the row: keys (k % NSUB) * SB.. of its (k / NSUB)-th block.
    auto issue = [&](int buf, int k) {
        const int p = p0 + k / NSUB, r0 = (k % NSUB) * SB;
        AsyncTile<D, SB>::issue(tk, smem + buf * BUF, K + (static_cast<size_t>(cols[p]) * BLK + r0) * D);
        AsyncTile<BLK, SB>::issue(ts, smem + buf * BUF + KT, dS + (static_cast<size_t>(p) * BLK + r0) * BLK);
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();
    const int nstage = (p1 - p0) * NSUB;
    if (nstage > 0) issue(0, 0);
    for (int k = 0; k < nstage; ++k) {
        const char *kt = smem + (k & 1) * BUF;
        const char *st = kt + KT;
        wait_vmcnt<0>();
        barrier_lds();  // this stage visible; every wave done with the other buffer
        if (k + 1 < nstage) issue((k + 1) & 1, k + 1);
#pragma unroll
        for (int kk = 0; kk < SB / O::KW; ++kk) {
            const typename O::frag b = Ts::frag_tr(st, kk * O::KW, 32 * w, lane);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[dt] = O::mma(Tk::frag_tr(kt, kk * O::KW, 32 * dt, lane), b, acc[dt]);
        }
    }

    if (slot < 0) {
        if constexpr (4 * 32 * D * 2 <= BUF) {
            // the buffer the last stage did not use; every wave is past it
            char *scratch = smem + (nstage & 1) * BUF + w * (32 * D * 2);
            store_tile_lds<D, DT>(scratch, static_cast<T *>(a.dq) + base + static_cast<size_t>(I * BLK + 32 * w) * D,
                                  acc, a.scale, lane);
        } else {
            store_rows<DT>(static_cast<T *>(a.dq) + base + static_cast<size_t>(I * BLK + 32 * w + li) * D, acc,
                           a.scale, lh);
        }
    } else {
        const size_t prow = (static_cast<size_t>(slot) * a.BH + bh) * BLK + 32 * w + li;
        store_rows<DT>(a.part + prow * D, acc, a.scale, lh);
    }
}

// Fixed-order sum of the partials of split lines: out rows of line L get
// sum_{s = 0..n-1} part[first + s]. Up to three jobs (dQ rows, dK and dV
// columns) share one launch; one workgroup per (job, merge, batch*head,
// 16-row slice).
struct SumJob {
    const int4 *merges;
    const float *part;
    void *out;
    int n;
};
struct SumArgs {
    SumJob job[3];
    int njobs, BH, S;
};

template <typename T, int D>
__global__ void __launch_bounds__(NT) sum_partials_kernel(SumArgs a) {
    constexpr int CH = D / 4;
    constexpr int MR = NT / CH;
    constexpr int SLICES = merge_slices<D>();
    int x = blockIdx.x;
    const int slice = x % SLICES;
    x /= SLICES;
    const int bh = x % a.BH;
    x /= a.BH;
    int j = 0;
    while (j < a.njobs - 1 && x >= a.job[j].n) x -= a.job[j++].n;
    const int4 mg = a.job[j].merges[x];
    const float *part = a.job[j].part;
    const int L = mg.x, s0 = mg.y, ns = mg.z;
    const int r = slice * MR + threadIdx.x / CH, c = threadIdx.x % CH;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = 0; s < ns; ++s) {
        const size_t pr = (static_cast<size_t>(s0 + s) * a.BH + bh) * BLK + r;
        const float4 v = *reinterpret_cast<const float4 *>(part + pr * D + 4 * c);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    T *dst = static_cast<T *>(a.job[j].out) + (static_cast<size_t>(bh) * a.S + L * BLK + r) * D + 4 * c;
    store4(dst, acc.x, acc.y, acc.z, acc.w);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------
// ---------------------------------------------------------------------------
// Block-sparse times dense, C = A B, on the same structure and plan (page
// "trnsparse 0.7.0 -> 0.9.0", CHANGELOG 0.8.0: only the stored blocks are
// visited, B is addressed by block column; CHANGELOG 0.9.0: output tiles
// balanced by stored blocks, one writer each). A is given by its stored
// 128 x 128 blocks in BSR order; B and C are dense [nb*128, n_cols].
// One workgroup per (row item, 128-column tile of C): for every stored block
// J of the row (or segment) and every KB-wide k slice of it, the A slice
// (128 x KB, rows 128 elements apart) and the B slice (KB x 128, rows n_cols
// apart) are staged in LDS, and C^T += B_slice^T A_slice^T on 32x32 MFMA
// tiles (lane = row of C). Split rows write fp32 shares, summed afterwards in
// a fixed order.
// ---------------------------------------------------------------------------
struct SpmmArgs {
    const void *blocks, *b;
    void *c;
    const int4 *items;
    const int32_t *col_idx;  // block row of B per entry (BSR: col_idx; transposed: BSC row_idx)
    const int32_t *a_block;  // transposed A only: the A block of each BSC entry (bsc_block)
    float *part;
    int n_cols, n_tiles, n_items;
    // Batches of problems over blockIdx.y (one per (batch, head) in the
    // wide-head attention path; 0 strides for a single product), in elements.
    size_t a_head, b_head, c_head, part_head;
    float mul;  // applied to C when it is written
};

constexpr int SPMM_NTILE = 128;  // C columns per workgroup

// Workgroups of an SpMM launch: the items padded to a multiple of 8, times
// the column tiles (see the item-to-XCD mapping in spmm_kernel).
inline unsigned spmm_blocks(int n_items, int n_tiles) {
    return static_cast<unsigned>((n_items + 7) / 8 * 8) * static_cast<unsigned>(n_tiles);
}

// TA: C = sum over the entries of a block column of A_q^T B_q (items are the
// BSC column items, A_q = blocks[a_block[q]]), the transposed products the
// wide-head backward needs for dK and dV.
// WPC: waves per 32 output rows. With 2 (16-bit operands) the workgroup has
// 8 waves, each computing half of the 128 columns of its 32 rows: two waves
// per SIMD when a launch has about one workgroup per CU (width 512 at
// n = 8192: 64 row items x 4 column tiles), so that one wave's operand waits
// are covered by the other's products.
template <typename T, int KB, int MINW, bool TA = false, int WPC = 1>
__global__ void __launch_bounds__(NT * WPC, MINW) spmm_kernel(SpmmArgs a) {
    using O = Op<T>;
    static_assert(!TA || sizeof(T) == 2, "transposed A for 16-bit operands only");
    static_assert(WPC == 1 || sizeof(T) == 2, "two waves per row group for 16-bit operands only");
    constexpr int NTH = NT * WPC;
    using Ta = std::conditional_t<TA, Tile<T, BLK>, Tile<T, KB>>;
    using Tb = Tile<T, SPMM_NTILE>;
    constexpr bool ASYNC = sizeof(T) == 2;
    constexpr int NBUF = ASYNC ? 2 : 1;
    constexpr int ATILE = BLK * KB * sizeof(T);
    constexpr int BTILE = KB * SPMM_NTILE * sizeof(T);
    constexpr int STAGE = ATILE + BTILE;
    constexpr int NSUB = BLK / KB;
    constexpr int KSK = KB / O::KW;
    constexpr int DT = SPMM_NTILE / 32 / WPC;  // 32-column tiles per wave
    __shared__ __attribute__((aligned(16))) char smem[NBUF * STAGE];

    const int tid = threadIdx.x, lane = tid & 63, li = lane & 31, lh = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), w = wave % 4, dt0 = (wave / 4) * DT;
    // The column tiles of one item go to one XCD (the dispatcher deals
    // consecutive workgroups to the 8 XCDs in turn): its A blocks are then
    // fetched into one L2 and hit there for the item's other tiles. Items
    // 8g .. 8g + 7 occupy workgroups [8 g n_tiles, 8 (g + 1) n_tiles).
    const int xcd = static_cast<int>(blockIdx.x % 8), rest = static_cast<int>(blockIdx.x / 8);
    const int tile = rest % a.n_tiles, item = (rest / a.n_tiles) * 8 + xcd;
    if (item >= a.n_items) return;  // padding of the last group of 8 items
    const int4 it = a.items[item];
    const int I = it.x, p0 = it.y, p1 = it.z, slot = it.w;
    const int n0 = tile * SPMM_NTILE;
    const size_t ldb = static_cast<size_t>(a.n_cols);
    const T *A = static_cast<const T *>(a.blocks) + blockIdx.y * a.a_head;
    const T *Bm = static_cast<const T *>(a.b) + blockIdx.y * a.b_head;
    const const_i32 *cols = as_const(a.col_idx);
    const int nstage = (p1 - p0) * NSUB;
    // A's k-slice of stage k: columns (k % NSUB) * KB.. of all 128 rows, or
    // with TA rows (k % NSUB) * KB.. (contiguous) of the entry's block.
    auto a_src = [&](int k) -> const T * {
        if constexpr (TA)
            return A + static_cast<size_t>(as_const(a.a_block)[p0 + k / NSUB]) * BLK * BLK + (k % NSUB) * KB * BLK;
        else
            return A + static_cast<size_t>(p0 + k / NSUB) * BLK * BLK + (k % NSUB) * KB;
    };
    auto b_src = [&](int k) -> const T * {
        return Bm + (static_cast<size_t>(cols[p0 + k / NSUB]) * BLK + (k % NSUB) * KB) * ldb + n0;
    };

    f32x16 acc[DT];
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] = zero16();

    if constexpr (ASYNC) {
        using CA = std::conditional_t<TA, AsyncTileStrided<BLK, KB, NTH>, AsyncTileStrided<KB, BLK, NTH>>;
        using CB = AsyncTileStrided<SPMM_NTILE, KB, NTH>;
        const uint32_t sa = BLK * sizeof(T), sbs = static_cast<uint32_t>(ldb * sizeof(T));
        const auto pa = CA::plan(tid, sa);
        const auto pb = CB::plan(tid, sbs);
        if (nstage > 0) {
            CA::issue(pa, smem, a_src(0), sa);
            CB::issue(pb, smem + ATILE, b_src(0), sbs);
        }
        for (int k = 0; k < nstage; ++k) {
            char *at = smem + (k & 1) * STAGE;
            char *bt = at + ATILE;
            wait_vmcnt<0>();
            barrier_lds();  // this stage visible; every wave done with the other buffer
            if (k + 1 < nstage) {
                char *na = smem + ((k + 1) & 1) * STAGE;
                CA::issue(pa, na, a_src(k + 1), sa);
                CB::issue(pb, na + ATILE, b_src(k + 1), sbs);
            }
#pragma unroll
            for (int kk = 0; kk < KSK; ++kk) {
                typename O::frag af;
                if constexpr (TA)
                    af = Ta::frag_tr(at, kk * O::KW, 32 * w, lane);
                else
                    af = Ta::frag_row(at, 32 * w + li, kk * O::KW + lh * O::KL);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    acc[dt] = O::mma(Tb::frag_tr(bt, kk * O::KW, 32 * (dt0 + dt), lane), af, acc[dt]);
            }
        }
    } else {
        for (int k = 0; k < nstage; ++k) {
            char *at = smem;
            char *bt = smem + ATILE;
            __syncthreads();
            Ta::template stage_strided<BLK>(at, a_src(k), BLK, tid);
            Tb::template stage_strided<KB>(bt, b_src(k), ldb, tid);
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < KSK; ++kk) {
                const typename O::frag af = Ta::frag_row(at, 32 * w + li, kk * O::KW + lh * O::KL);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
                    acc[dt] = O::mma(Tb::frag_tr(bt, kk * O::KW, 32 * dt, lane), af, acc[dt]);
            }
        }
    }

    const int r = 32 * w + li;
    const int c0 = n0 + 32 * dt0;
    if (slot < 0) {
        store_rows<DT>(static_cast<T *>(a.c) + blockIdx.y * a.c_head + (static_cast<size_t>(I) * BLK + r) * ldb + c0,
                       acc, a.mul, lh);
    } else {
        store_rows<DT>(a.part + blockIdx.y * a.part_head + (static_cast<size_t>(slot) * BLK + r) * ldb + c0, acc,
                       a.mul, lh);
    }
}

// Fixed-order sum of the shares of split rows: C rows of line L get
// sum_{s = 0..n-1} part[first + s]; one thread per 4 columns of a row.
template <typename T>
__global__ void __launch_bounds__(NT) spmm_sum_kernel(const int4 *merges, const float *part, void *c, int n_cols,
                                                      int chunks_per_merge, size_t part_head, size_t c_head) {
    part += blockIdx.y * part_head;
    c = static_cast<T *>(c) + blockIdx.y * c_head;
    const int mi = blockIdx.x / chunks_per_merge;
    const int64_t id = static_cast<int64_t>(blockIdx.x % chunks_per_merge) * NT + threadIdx.x;
    const int cols4 = n_cols / 4;
    if (id >= static_cast<int64_t>(BLK) * cols4) return;
    const int r = static_cast<int>(id / cols4), c4 = static_cast<int>(id % cols4);
    const int4 mg = merges[mi];
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int s = 0; s < mg.z; ++s) {
        const float4 v = *reinterpret_cast<const float4 *>(part + (static_cast<size_t>(mg.y + s) * BLK + r) * n_cols + 4 * c4);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
    }
    store4(static_cast<T *>(c) + (static_cast<size_t>(mg.x) * BLK + r) * n_cols + 4 * c4, acc.x, acc.y, acc.z, acc.w);
}

// ---------------------------------------------------------------------------
// Wide heads (head_dim 512). The forward runs the fused kernels in their
// two-pass form (statistics, then output with P already normalised): with one
// wave per SIMD the 32 x 512 fp32 output accumulator fits the matrix unit's
// 256 registers, and the output pass never rescales it. In the backward the
// dQ and dK/dV accumulators do not fit next to their operands, so the
// gradient blocks are materialised: P and dS = P (dP - delta) per stored
// block from S and dP = dO V^T computed together (sddmm_bwd), then
// dQ = scale dS K (spmm), dV = P^T dO and dK = scale dS^T Q (spmm with
// transposed blocks, column-first over the BSC order). Blocks are
// [BH][nnzb][128][128] in BSR order, in the operand dtype.
// ---------------------------------------------------------------------------
// Backward score blocks, both products of a block in one pass: for each
// stored block p of a row item, S^T = K_J Q_I^T and dP^T = V_J dO_I^T with
// lane = query (the contraction over D in 64-wide slices; K, V and dO staged
// by LDS-DMA, Q held in registers), and in the epilogue P = 2^(S*c - lse2) and
// dS = P (dP - delta) in the operand dtype, row-major by query (the layout
// the block products read). Neither S nor dP goes through memory. Each lane
// holds four runs of four consecutive keys of its query, stored 8 bytes at a
// time.
struct SddmmBwdArgs {
    const void *q, *k, *dout, *v;  // [BH][S][D]
    void *p, *ds;                  // [BH][nnzb][128][128], operand dtype
    const float *lse2, *delta;     // [BH][S]: base-2 log-sum-exp; delta stored negated
    const int4 *items;             // row items: {block row, first, end, slot}
    const int32_t *col_idx;
    int BH, S, nnzb;
    float c;  // scale * log2(e)
};

template <typename T, int D>
__global__ void __launch_bounds__(NT) sddmm_bwd_kernel(SddmmBwdArgs a) {
    using O = Op<T>;
    using Tl = Tile<T, 64>;
    static_assert(sizeof(T) == 2, "16-bit operands only");
    constexpr int KC = 64;            // contraction slice
    constexpr int SL = BLK * KC * 2;  // one operand slice (16 KB)
    constexpr int NK = D / KC;        // slices per block
    constexpr int KSL = KC / O::KW;   // k-steps per slice
    static_assert(NK % 2 == 0, "slice buffers alternate within a block");
    __shared__ __attribute__((aligned(16))) char smem[2 * 3 * SL];
    using C = AsyncTileStrided<KC, BLK>;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 31, lh = lane >> 5;
    const int4 it = a.items[blockIdx.x];
    const int I = it.x, p0 = it.y, p1 = it.z;
    const int bh = blockIdx.y;
    const size_t base = static_cast<size_t>(bh) * a.S * D;
    const size_t rows_i = base + static_cast<size_t>(I) * BLK * D;
    const T *dOi = static_cast<const T *>(a.dout) + rows_i;
    const T *K = static_cast<const T *>(a.k) + base, *V = static_cast<const T *>(a.v) + base;
    const const_i32 *cols = as_const(a.col_idx);
    const uint32_t stride = D * 2;
    const auto pl = C::plan(tid, stride);
    const int nblk = p1 - p0;
    // slice kc of block pb: K and V of its key block, dO of the row's queries
    auto issue = [&](int pb, int kc) {
        char *buf = smem + (kc & 1) * 3 * SL;
        const size_t kr = static_cast<size_t>(cols[p0 + pb]) * BLK * D + kc * KC;
        C::issue(pl, buf, K + kr, stride);
        C::issue(pl, buf + SL, dOi + kc * KC, stride);
        C::issue(pl, buf + 2 * SL, V + kr, stride);
    };
    const int qrow = 32 * w + li;  // this lane's query row of the block row
    const size_t srow = static_cast<size_t>(bh) * a.S + static_cast<size_t>(I) * BLK + qrow;
    const float lse = a.lse2[srow], dl = a.delta[srow];
    if (nblk > 0) issue(0, 0);
    // The lane's Q row stays in registers for the whole item (128 per lane):
    // only K, V and dO go through LDS, for every block.
    typename O::frag qf[NK * KSL];
    if (nblk > 0) {
        const T *qr = static_cast<const T *>(a.q) + rows_i + static_cast<size_t>(qrow) * D + lh * O::KL;
#pragma unroll
        for (int g = 0; g < NK * KSL; ++g) qf[g] = gfrag(qr + g * O::KW);
    }
    // One block per outer iteration; its slices unrolled (buffer kc & 1), so
    // the accumulators stay in the matrix unit's registers and the Q
    // fragments are indexed by constants.
    for (int pb = 0; pb < nblk; ++pb) {
        f32x16 sc[4], dp[4];  // key tiles j: S^T and dP^T, lane = query
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            sc[j] = zero16();
            dp[j] = zero16();
        }
#pragma unroll
        for (int kc = 0; kc < NK; ++kc) {
            const char *kt = smem + (kc & 1) * 3 * SL, *ot = kt + SL, *vt = kt + 2 * SL;
            wait_vmcnt<0>();
            barrier_lds();  // this slice visible; every wave done with the other buffer
            if (kc + 1 < NK) issue(pb, kc + 1);
            else if (pb + 1 < nblk) issue(pb + 1, 0);
#pragma unroll
            for (int ks = 0; ks < KSL; ++ks) {
                const int c0 = ks * O::KW + lh * O::KL;
                const typename O::frag of = Tl::frag_row(ot, qrow, c0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sc[j] = O::mma(Tl::frag_row(kt, 32 * j + li, c0), qf[kc * KSL + ks], sc[j]);
                    dp[j] = O::mma(Tl::frag_row(vt, 32 * j + li, c0), of, dp[j]);
                }
            }
        }
        {
            // value v of tile j: key 32j + 8(v/4) + 4(lane/32) + v%4 of query qrow
            const size_t at = ((static_cast<size_t>(bh) * a.nnzb + p0 + pb) * BLK + qrow) * BLK + 4 * lh;
            T *prow = static_cast<T *>(a.p) + at, *dsrow = static_cast<T *>(a.ds) + at;
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float pv[4], dv[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        pv[e] = exp2_fast(fmaf(sc[j][4 * g + e], a.c, -lse));
                        dv[e] = pv[e] * (dp[j][4 * g + e] + dl);
                    }
                    store4(prow + 32 * j + 8 * g, pv[0], pv[1], pv[2], pv[3]);
                    store4(dsrow + 32 * j + 8 * g, dv[0], dv[1], dv[2], dv[3]);
                }
        }
    }
}

struct PlanView {
    const int32_t *col_idx, *row_idx, *row_ptr, *bsc_block;
    const int32_t *row_queues[kQueueLevels], *col_queues[kQueueLevels];
    const int4 *row_items, *col_items, *row_merges, *col_merges;
};

PlanView view(const bsr_attn_structure &s, const int32_t *d_plan) {
    const std::vector<int32_t> &h = s.plan;
    PlanView v;
    v.col_idx = d_plan + h[H_OFF_COL_IDX];
    v.row_idx = d_plan + h[H_OFF_ROW_IDX];
    v.row_ptr = d_plan + h[H_OFF_ROW_PTR];
    v.bsc_block = d_plan + h[H_OFF_BSC_BLOCK];
    for (int lv = 0; lv < kQueueLevels; ++lv) {
        v.row_queues[lv] = d_plan + h[h[H_OFF_ROW_SCHED] + lv];
        v.col_queues[lv] = d_plan + h[h[H_OFF_COL_SCHED] + lv];
    }
    v.row_items = reinterpret_cast<const int4 *>(d_plan + h[H_OFF_ROW_ITEMS]);
    v.col_items = reinterpret_cast<const int4 *>(d_plan + h[H_OFF_COL_ITEMS]);
    v.row_merges = reinterpret_cast<const int4 *>(d_plan + h[H_OFF_ROW_MERGES]);
    v.col_merges = reinterpret_cast<const int4 *>(d_plan + h[H_OFF_COL_MERGES]);
    return v;
}

// Row repacking between head dims (a head dim without an instance of its
// own runs on the next instantiated width): every row of `rows` is copied
// from src (src_chunks 16-byte chunks per row) to dst (dst_chunks per row);
// columns past the source row are zero-filled, columns past the destination
// row dropped. Up to five tensors of the same shape per launch (blockIdx.y).
struct RepackArgs {
    const int4 *src[5];
    int4 *dst[5];
    int64_t rows;
    int src_chunks, dst_chunks;
};

__global__ void __launch_bounds__(NT) repack_kernel(RepackArgs a) {
    const int4 *src = a.src[blockIdx.y];
    int4 *dst = a.dst[blockIdx.y];
    const int64_t total = a.rows * a.dst_chunks;
    const int64_t step = static_cast<int64_t>(gridDim.x) * NT;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * NT + threadIdx.x; i < total; i += step) {
        const int64_t r = i / a.dst_chunks;
        const int c = static_cast<int>(i - r * a.dst_chunks);
        dst[i] = c < a.src_chunks ? src[r * a.src_chunks + c] : make_int4(0, 0, 0, 0);
    }
}

// MFMA-loop probe: the sustained matrix-core rate on this device with
// random operands (the rate is power-limited and depends on the data). Each
// wave runs CHAINS independent accumulations of `iters` products on register
// operands drawn from a per-lane hash; nothing is read, and the sum is
// written to sink[0] only if it equals a value it never takes, so the work
// cannot be removed.
template <typename T>
__global__ void __launch_bounds__(NT, 2) mfma_probe_kernel(int iters, float *sink) {
    using O = Op<T>;
    constexpr int CHAINS = 4;
    uint32_t h = (blockIdx.x * NT + threadIdx.x) * 2654435761u + 12345u;
    auto next = [&]() {  // xorshift32, uniform in (-1, 1)
        h ^= h << 13;
        h ^= h >> 17;
        h ^= h << 5;
        return static_cast<float>(static_cast<int32_t>(h)) * (1.f / 2147483648.f);
    };
    typename O::frag a[CHAINS], b[CHAINS];
    f32x16 acc[CHAINS];
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int e = 0; e < O::KL; ++e) {
                a[c][e] = static_cast<T>(next());
                b[c][e] = static_cast<T>(next());
            }
        } else {
            a[c] = next();
            b[c] = next();
        }
        acc[c] = zero16();
    }
    for (int i = 0; i < iters; ++i)
#pragma unroll
        for (int c = 0; c < CHAINS; ++c) acc[c] = O::mma(a[c], b[c], acc[c]);
    float total = 0.f;
#pragma unroll
    for (int c = 0; c < CHAINS; ++c)
#pragma unroll
        for (int v = 0; v < 16; ++v) total += acc[c][v];
    if (total == 1234.5678f) sink[0] = total;
}

// Staged sub-block rows and the waves-per-SIMD target of each kernel. Every
// stage is double-buffered (LDS-DMA; fp32 tiles in 16-byte chunks, TileF4).
// 16-bit fwd and dQ use 64-row sub-blocks: 64 KB of LDS and two workgroups
// per CU at D <= 128, 128 KB and one workgroup per CU at D = 256 (32-row
// sub-blocks there measured 20 % slower in the forward: twice the barriers
// and copy issues per product). dK/dV holds K, V and both accumulators in
// registers, so it runs one workgroup per CU with 128-row sub-blocks. fp32
// runs one workgroup per CU (its fragments take one register per element).
template <typename T, int D> struct Launch {
    static constexpr bool BF = sizeof(T) == 2;
    static constexpr int FWD_SB = BF ? (D >= 512 ? 32 : 64) : (D >= 128 ? 64 : 128);
    static constexpr int DQ_SB = BF ? 64 : (D >= 128 ? 32 : 64);
    static constexpr int DKDV_SB = D >= 128 ? 64 : 128;  // dkdv_kernel (fp32)
    static constexpr int FWD_W = (BF && D <= 128) ? 2 : 1;
    static constexpr int DQ_W = (BF && D <= 128) ? 2 : 1;
    static constexpr int DKDV_W = 1;
    // dK/dV through per-head work queues (whole 128-row stages) where the
    // K and V tiles fit one stage buffer; at head_dim 128 with two waves per
    // SIMD that split each tile's work by role (dkdv_pair_kernel).
    static constexpr bool DKDV_QUEUES = BF && D <= 128;
    static constexpr bool DKDV_PAIR = BF && D == 128;
    // dK/dV at head dim 256 over two waves per SIMD split by role
    // (dkdv_wide_pair_kernel).
    static constexpr bool DKDV_WIDE_PAIR = BF && D == 256;
    // Forward split by role over two waves per SIMD (fwd_pair_kernel) at head
    // dim 256, where the one-wave forward holds Q and the accumulator together
    // (C4 forward 86.5 -> 77.8 us). At 128 the one-wave forward already runs
    // two workgroups, so two waves, per SIMD; the pair form there is one
    // workgroup per CU and measured slower (C3 forward 50.5 -> 67 us).
    static constexpr bool FWD_PAIR = BF && D == 256;
    // dQ split the same way at head dim 256 (C4 dQ 117.6 -> 108.3 us).
    static constexpr bool DQ_PAIR = BF && D == 256;
    static constexpr int DKDV_QUEUE_WGS_PER_CU = D <= 64 ? 2 : 1;  // LDS: 66 KB or 130 KB
    // dQ from stored dS: 64-key stages of K and dS^T (64 KB of LDS at D = 128)
    static constexpr int DQ_DS_SB = 64;
    static constexpr int DQ_DS_W = D <= 128 ? 2 : 1;
};

// Compute units of the current device (cached per device).
int compute_units() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Largest queue level lv (2^lv queues per head, lv < kQueueLevels) with
// 2^lv * BH workgroups fitting `slots` concurrent workgroups; at least 0.
int queue_level(int BH, int slots) {
    int lv = 0;
    while (lv + 1 < kQueueLevels && (static_cast<int64_t>(BH) << (lv + 1)) <= slots) ++lv;
    return lv;
}

template <typename T, int D>
int fwd_impl(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o, float *row_max,
             float *row_denom, void *ws) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    FwdWorkspace wl = fwd_workspace(s, c.BH, D);
    char *w = static_cast<char *>(ws);
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.row_max = row_max; a.row_denom = row_denom;
    a.items = pv.row_items; a.col_idx = pv.col_idx;
    a.part_o = w ? reinterpret_cast<float *>(w + wl.part_o) : nullptr;
    a.part_m2 = w ? reinterpret_cast<float *>(w + wl.part_m2) : nullptr;
    a.part_l = w ? reinterpret_cast<float *>(w + wl.part_l) : nullptr;
    a.part_mx = w ? reinterpret_cast<float *>(w + wl.part_mx) : nullptr;
    a.BH = c.BH; a.S = c.S;
    a.c = c.scale * LOG2E;
    const unsigned grid = static_cast<unsigned>(s.row_items.size()) * c.BH;
    {
        KernelTimer tm("fwd", dtype_name<T>(), D, st);
        if constexpr (Launch<T, D>::FWD_PAIR)
            hipLaunchKernelGGL((fwd_pair_kernel<T, D>), dim3(grid), dim3(NT2), 0, st, a);
        else
            hipLaunchKernelGGL((fwd_kernel<T, D, Launch<T, D>::FWD_SB, Launch<T, D>::FWD_W, FWD_ONE_PASS>), dim3(grid),
                               dim3(NT), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (!s.row_merges.empty()) {
        MergeArgs m;
        m.merges = pv.row_merges;
        m.part_o = a.part_o; m.part_m2 = a.part_m2; m.part_l = a.part_l; m.part_mx = a.part_mx;
        m.o = o; m.row_max = row_max; m.row_denom = row_denom;
        m.BH = c.BH; m.S = c.S;
        const unsigned g2 = static_cast<unsigned>(s.row_merges.size()) * c.BH * merge_slices<D>();
        KernelTimer tm("fwd_merge", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((fwd_merge_kernel<T, D, true>), dim3(g2), dim3(NT), 0, st, m);
        e = hipGetLastError();
    }
    return e;
}

// Two-pass forward (statistics, then output): four launches where the
// one-pass forward needs two; kept as the pages' variant for comparison.
template <typename T, int D>
int fwd_two_pass_impl(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o, float *row_max,
                      float *row_denom, void *ws) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    FwdWorkspace wl = fwd_workspace(s, c.BH, D);
    char *w = static_cast<char *>(ws);
    FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o;
    a.row_max = row_max; a.row_denom = row_denom;
    a.items = pv.row_items; a.col_idx = pv.col_idx;
    a.part_o = w ? reinterpret_cast<float *>(w + wl.part_o) : nullptr;
    a.part_m2 = w ? reinterpret_cast<float *>(w + wl.part_m2) : nullptr;
    a.part_l = w ? reinterpret_cast<float *>(w + wl.part_l) : nullptr;
    a.part_mx = w ? reinterpret_cast<float *>(w + wl.part_mx) : nullptr;
    a.BH = c.BH; a.S = c.S;
    a.c = c.scale * LOG2E;
    const unsigned grid = static_cast<unsigned>(s.row_items.size()) * c.BH;
    constexpr int SB = Launch<T, D>::FWD_SB, W = Launch<T, D>::FWD_W;
    hipError_t e;
    {
        KernelTimer tm("fwd_stats", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((fwd_kernel<T, D, SB, W, FWD_STATS>), dim3(grid), dim3(NT), 0, st, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!s.row_merges.empty()) {
        MergeArgs m;
        m.merges = pv.row_merges;
        m.part_o = a.part_o; m.part_m2 = a.part_m2; m.part_l = a.part_l; m.part_mx = a.part_mx;
        m.o = o; m.row_max = row_max; m.row_denom = row_denom;
        m.BH = c.BH; m.S = c.S;
        const unsigned g2 = static_cast<unsigned>(s.row_merges.size()) * c.BH * merge_slices<D>();
        KernelTimer tm("fwd_merge_stats", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((fwd_merge_kernel<T, D, false>), dim3(g2), dim3(NT), 0, st, m);
        if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    {
        KernelTimer tm("fwd_out", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((fwd_kernel<T, D, SB, W, FWD_OUT>), dim3(grid), dim3(NT), 0, st, a);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if (!s.row_merges.empty()) {
        SumArgs sa{};
        sa.job[sa.njobs++] = SumJob{pv.row_merges, a.part_o, o, static_cast<int>(s.row_merges.size())};
        sa.BH = c.BH;
        sa.S = c.S;
        KernelTimer tm("sum_partials", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((sum_partials_kernel<T, D>),
                           dim3(static_cast<unsigned>(s.row_merges.size()) * c.BH * merge_slices<D>()), dim3(NT), 0,
                           st, sa);
        e = hipGetLastError();
    }
    return e;
}

template <typename T>
int spmm_impl(const SpmmCommon &c, const void *blocks, const void *b, void *cm, void *ws) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    constexpr int KB = sizeof(T) == 2 ? 64 : 32;
    constexpr int W = sizeof(T) == 2 ? 2 : 1;
    SpmmArgs a;
    a.blocks = blocks; a.b = b; a.c = cm;
    a.items = pv.row_items; a.col_idx = pv.col_idx; a.a_block = nullptr;
    a.part = static_cast<float *>(ws);
    a.a_head = a.b_head = a.c_head = a.part_head = 0;
    a.mul = 1.f;
    // (64-column tiles, which double the grid on small problems, measured
    // slower: every extra workgroup re-reads its A slices.)
    a.n_cols = c.n_cols;
    a.n_tiles = c.n_cols / SPMM_NTILE;
    a.n_items = static_cast<int>(s.row_items.size());
    {
        KernelTimer tm("spmm", dtype_name<T>(), 0, st);
        constexpr int WPC = sizeof(T) == 2 ? 2 : 1;
        hipLaunchKernelGGL((spmm_kernel<T, KB, W, false, WPC>), dim3(spmm_blocks(a.n_items, a.n_tiles)),
                           dim3(NT * WPC), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || s.row_merges.empty()) return e;
    const int chunks = static_cast<int>((static_cast<int64_t>(BLK) * (c.n_cols / 4) + NT - 1) / NT);
    KernelTimer tm("spmm_sum", dtype_name<T>(), 0, st);
    hipLaunchKernelGGL((spmm_sum_kernel<T>), dim3(static_cast<unsigned>(s.row_merges.size()) * chunks), dim3(NT), 0,
                       st, pv.row_merges, a.part, cm, c.n_cols, chunks, size_t{0}, size_t{0});
    return hipGetLastError();
}

// The dK/dV pass (DS: also store dS for the dQ pass that reads it).
template <typename T, int D, bool DS>
hipError_t launch_dkdv(const LaunchCommon &c, const PlanView &pv, DkdvArgs &ka) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    if constexpr (Launch<T, D>::DKDV_PAIR) {
        // one 512-thread workgroup per CU
        const int lv = queue_level(c.BH, compute_units());
        ka.queues = pv.col_queues[lv];
        ka.n_queues = 1 << lv;
        KernelTimer tm(DS ? "dkdv_ds" : "dkdv", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((dkdv_pair_kernel<T, D, DS>), dim3(static_cast<unsigned>(ka.n_queues) * c.BH), dim3(NT2),
                           0, st, ka);
    } else if constexpr (Launch<T, D>::DKDV_WIDE_PAIR) {
        KernelTimer tm(DS ? "dkdv_ds" : "dkdv", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((dkdv_wide_pair_kernel<T, D, DS>), dim3(static_cast<unsigned>(s.col_items.size()) * c.BH),
                           dim3(NT2), 0, st, ka);
    } else if constexpr (Launch<T, D>::DKDV_QUEUES) {
        // as many queues per head as fill the CUs
        const int lv = queue_level(c.BH, compute_units() * Launch<T, D>::DKDV_QUEUE_WGS_PER_CU);
        ka.queues = pv.col_queues[lv];
        ka.n_queues = 1 << lv;
        KernelTimer tm(DS ? "dkdv_ds" : "dkdv", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((dkdv_queue_kernel<T, D, DS>), dim3(static_cast<unsigned>(ka.n_queues) * c.BH), dim3(NT),
                           0, st, ka);
    } else {
        KernelTimer tm(DS ? "dkdv_ds" : "dkdv", dtype_name<T>(), D, st);
        static_assert(!DS, "the dS-storing schedule takes 16-bit operands");
        hipLaunchKernelGGL((dkdv_kernel<T, D, Launch<T, D>::DKDV_SB, Launch<T, D>::DKDV_W>),
                           dim3(static_cast<unsigned>(s.col_items.size()) * c.BH), dim3(NT), 0, st, ka);
    }
    return hipGetLastError();
}

// Fixed-order sums of the dQ, dK and dV partials of split lines.
template <typename T, int D>
hipError_t launch_backward_sums(const LaunchCommon &c, const PlanView &pv, float *pdq, float *pdk, float *pdv,
                                void *dq, void *dk, void *dv) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    SumArgs sa{};
    int total = 0;
    if (!s.row_merges.empty()) {
        sa.job[sa.njobs++] = SumJob{pv.row_merges, pdq, dq, static_cast<int>(s.row_merges.size())};
        total += static_cast<int>(s.row_merges.size());
    }
    if (!s.col_merges.empty()) {
        sa.job[sa.njobs++] = SumJob{pv.col_merges, pdk, dk, static_cast<int>(s.col_merges.size())};
        sa.job[sa.njobs++] = SumJob{pv.col_merges, pdv, dv, static_cast<int>(s.col_merges.size())};
        total += 2 * static_cast<int>(s.col_merges.size());
    }
    if (sa.njobs == 0) return hipSuccess;
    sa.BH = c.BH;
    sa.S = c.S;
    KernelTimer tm("sum_partials", dtype_name<T>(), D, st);
    hipLaunchKernelGGL((sum_partials_kernel<T, D>), dim3(static_cast<unsigned>(total) * c.BH * merge_slices<D>()),
                       dim3(NT), 0, st, sa);
    return hipGetLastError();
}

template <typename T, int D>
DkdvArgs dkdv_args(const LaunchCommon &c, const PlanView &pv, const void *q, const void *k, const void *v,
                   const void *d_o, const float *delta, const float *lse2, void *dk, void *dv, float *pdk,
                   float *pdv) {
    DkdvArgs ka{};
    ka.q = q; ka.k = k; ka.v = v; ka.dout = d_o;
    ka.delta = delta; ka.lse2 = lse2; ka.dk = dk; ka.dv = dv;
    ka.items = pv.col_items; ka.row_idx = pv.row_idx; ka.part_dk = pdk; ka.part_dv = pdv;
    ka.BH = c.BH; ka.S = c.S; ka.c = c.scale * LOG2E; ka.scale = c.scale;
    ka.queues = nullptr; ka.n_queues = 0;
    ka.ds = nullptr; ka.bsc_block = pv.bsc_block; ka.nnzb = c.s->nnzb;
    return ka;
}

template <typename T, int D>
int bwd_impl(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o, const void *d_o,
             const float *row_max, const float *row_denom, void *dq, void *dk, void *dv, void *ws) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    BwdWorkspace wl = bwd_workspace(s, c.BH, c.S, D);
    char *w = static_cast<char *>(ws);
    float *delta = reinterpret_cast<float *>(w + wl.delta);
    float *lse2 = reinterpret_cast<float *>(w + wl.lse2);
    float *pdq = reinterpret_cast<float *>(w + wl.part_dq);
    float *pdk = reinterpret_cast<float *>(w + wl.part_dk);
    float *pdv = reinterpret_cast<float *>(w + wl.part_dv);

    hipError_t e;
    DqArgs qa;
    qa.q = q; qa.k = k; qa.v = v; qa.o = o; qa.dout = d_o;
    qa.row_max = row_max; qa.row_denom = row_denom;
    qa.delta = delta; qa.lse2 = lse2; qa.dq = dq;
    qa.items = pv.row_items; qa.col_idx = pv.col_idx; qa.row_ptr = pv.row_ptr; qa.part = pdq;
    qa.BH = c.BH; qa.S = c.S; qa.c = c.scale * LOG2E; qa.scale = c.scale;
    {
        KernelTimer tm("dq", dtype_name<T>(), D, st);
        if constexpr (Launch<T, D>::DQ_PAIR)
            hipLaunchKernelGGL((dq_pair_kernel<T, D>), dim3(static_cast<unsigned>(s.row_items.size()) * c.BH),
                               dim3(NT2), 0, st, qa);
        else
            hipLaunchKernelGGL((dq_kernel<T, D, Launch<T, D>::DQ_SB, Launch<T, D>::DQ_W>),
                               dim3(static_cast<unsigned>(s.row_items.size()) * c.BH), dim3(NT), 0, st, qa);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    DkdvArgs ka = dkdv_args<T, D>(c, pv, q, k, v, d_o, delta, lse2, dk, dv, pdk, pdv);
    if ((e = launch_dkdv<T, D, false>(c, pv, ka)) != hipSuccess) return e;
    return launch_backward_sums<T, D>(c, pv, pdq, pdk, pdv, dq, dk, dv);
}

// The dS-storing backward: row terms, then dK/dV storing dS (bf16/fp16, in the
// workspace after the backward's own carve-up), then dQ = scale * dS K from
// the stored dS, then the partial sums.
template <typename T, int D>
int bwd_ds_impl(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o, const void *d_o,
                const float *row_max, const float *row_denom, void *dq, void *dk, void *dv, void *ws) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    BwdWorkspace wl = bwd_workspace(s, c.BH, c.S, D);
    char *w = static_cast<char *>(ws);
    float *delta = reinterpret_cast<float *>(w + wl.delta);
    float *lse2 = reinterpret_cast<float *>(w + wl.lse2);
    float *pdq = reinterpret_cast<float *>(w + wl.part_dq);
    float *pdk = reinterpret_cast<float *>(w + wl.part_dk);
    float *pdv = reinterpret_cast<float *>(w + wl.part_dv);
    void *dsbuf = w + ds_offset(wl.total);

    hipError_t e;
    PrepArgs pa{o, d_o, row_max, row_denom, delta, lse2, static_cast<int64_t>(c.BH) * c.S};
    {
        constexpr int rows_per_block = NT / (D / 8) * 4;
        KernelTimer tm("prep", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((prep_kernel<T, D>),
                           dim3(static_cast<unsigned>((pa.rows + rows_per_block - 1) / rows_per_block)), dim3(NT), 0,
                           st, pa);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;

    DkdvArgs ka = dkdv_args<T, D>(c, pv, q, k, v, d_o, delta, lse2, dk, dv, pdk, pdv);
    ka.ds = dsbuf;
    if ((e = launch_dkdv<T, D, true>(c, pv, ka)) != hipSuccess) return e;

    DqDsArgs qa{k, dsbuf, dq, pv.row_items, pv.col_idx, pdq, c.BH, c.S, s.nnzb, c.scale};
    {
        KernelTimer tm("dq_ds", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((dq_ds_kernel<T, D, Launch<T, D>::DQ_DS_SB, Launch<T, D>::DQ_DS_W>),
                           dim3(static_cast<unsigned>(s.row_items.size()) * c.BH), dim3(NT), 0, st, qa);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    return launch_backward_sums<T, D>(c, pv, pdq, pdk, pdv, dq, dk, dv);
}

// Block-sparse products of the wide-head path over every (batch, head):
// C = mul * (A B) row-first over the BSR items (trans = false), or
// C = mul * (A^T B) column-first over the BSC items (trans = true); split
// lines through fp32 partials summed in a fixed order.
template <typename T, int D>
hipError_t wide_spmm(const LaunchCommon &c, const PlanView &pv, bool trans, const void *blocks, const void *b,
                     void *out, float *part, float mul) {
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    SpmmArgs a{};
    a.blocks = blocks; a.b = b; a.c = out;
    a.items = trans ? pv.col_items : pv.row_items;
    a.col_idx = trans ? pv.row_idx : pv.col_idx;
    a.a_block = pv.bsc_block;
    a.part = part;
    a.n_cols = D;
    a.n_tiles = D / SPMM_NTILE;
    a.a_head = static_cast<size_t>(s.nnzb) * BLK * BLK;
    a.b_head = a.c_head = static_cast<size_t>(c.S) * D;
    a.part_head = static_cast<size_t>(trans ? s.n_col_slots : s.n_row_slots) * BLK * D;
    a.mul = mul;
    a.n_items = static_cast<int>(trans ? s.col_items.size() : s.row_items.size());
    {
        KernelTimer tm(trans ? "wide_spmm_t" : "wide_spmm", dtype_name<T>(), D, st);
        const dim3 grid(spmm_blocks(a.n_items, a.n_tiles), c.BH);
        if (trans)
            hipLaunchKernelGGL((spmm_kernel<T, 64, 2, true>), grid, dim3(NT), 0, st, a);
        else
            hipLaunchKernelGGL((spmm_kernel<T, 64, 2, false>), grid, dim3(NT), 0, st, a);
    }
    hipError_t e = hipGetLastError();
    const size_t n_merges = trans ? s.col_merges.size() : s.row_merges.size();
    if (e != hipSuccess || n_merges == 0) return e;
    const int chunks = (BLK * (D / 4) + NT - 1) / NT;
    KernelTimer tm("wide_spmm_sum", dtype_name<T>(), D, st);
    hipLaunchKernelGGL((spmm_sum_kernel<T>), dim3(static_cast<unsigned>(n_merges) * chunks, c.BH), dim3(NT), 0, st,
                       trans ? pv.col_merges : pv.row_merges, part, out, D, chunks, a.part_head, a.c_head);
    return hipGetLastError();
}

// Wide-head backward: delta and lse2, the P and dS blocks, then
// dQ = scale dS K, dV = P^T dO, dK = scale dS^T Q.
template <typename T>
int bwd_wide_impl(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o, const void *d_o,
                  const float *row_max, const float *row_denom, void *dq, void *dk, void *dv, void *ws) {
    constexpr int D = 512;
    const bsr_attn_structure &s = *c.s;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    PlanView pv = view(s, c.d_plan);
    const WideWorkspace wl = wide_workspace(s, c.BH, c.S, D, sizeof(T));
    char *w = static_cast<char *>(ws);
    float *delta = reinterpret_cast<float *>(w + wl.delta);
    float *lse2 = reinterpret_cast<float *>(w + wl.lse2);
    void *pb = w + wl.p;
    void *dsb = w + wl.ds;
    float *prow = reinterpret_cast<float *>(w + wl.part_rows);
    float *pcol = reinterpret_cast<float *>(w + wl.part_cols);
    hipError_t e;
    PrepArgs pa{o, d_o, row_max, row_denom, delta, lse2, static_cast<int64_t>(c.BH) * c.S};
    {
        constexpr int rows_per_block = NT / (D / 8) * 4;
        KernelTimer tm("prep", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((prep_kernel<T, D>),
                           dim3(static_cast<unsigned>((pa.rows + rows_per_block - 1) / rows_per_block)), dim3(NT), 0,
                           st, pa);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    SddmmBwdArgs ba{q, k, d_o, v, pb, dsb, lse2, delta, pv.row_items, pv.col_idx, c.BH, c.S, s.nnzb,
                    c.scale * LOG2E};
    {
        KernelTimer tm("sddmm_bwd", dtype_name<T>(), D, st);
        hipLaunchKernelGGL((sddmm_bwd_kernel<T, D>), dim3(static_cast<unsigned>(s.row_items.size()), c.BH), dim3(NT),
                           0, st, ba);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = wide_spmm<T, D>(c, pv, false, dsb, k, dq, prow, c.scale)) != hipSuccess) return e;
    if ((e = wide_spmm<T, D>(c, pv, true, pb, d_o, dv, pcol, 1.f)) != hipSuccess) return e;
    return wide_spmm<T, D>(c, pv, true, dsb, q, dk, pcol, c.scale);
}

int launch_fwd_at(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o, float *row_max,
                  float *row_denom, void *ws) {
    if (c.dtype == BSR_ATTN_F16) {
        switch (c.D) {
            case 32: return fwd_impl<_Float16, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_impl<_Float16, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_impl<_Float16, 128>(c, q, k, v, o, row_max, row_denom, ws);
            case 256: return fwd_impl<_Float16, 256>(c, q, k, v, o, row_max, row_denom, ws);
            case 512: return fwd_two_pass_impl<_Float16, 512>(c, q, k, v, o, row_max, row_denom, ws);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.dtype == BSR_ATTN_BF16) {
        switch (c.D) {
            case 32: return fwd_impl<__bf16, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_impl<__bf16, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_impl<__bf16, 128>(c, q, k, v, o, row_max, row_denom, ws);
            case 256: return fwd_impl<__bf16, 256>(c, q, k, v, o, row_max, row_denom, ws);
            case 512: return fwd_two_pass_impl<__bf16, 512>(c, q, k, v, o, row_max, row_denom, ws);
        }
    } else {
        switch (c.D) {
            case 32: return fwd_impl<float, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_impl<float, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_impl<float, 128>(c, q, k, v, o, row_max, row_denom, ws);
        }
    }
    return hipErrorInvalidValue;
}

int launch_fwd_two_pass_at(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o,
                           float *row_max, float *row_denom, void *ws) {
    if (c.dtype == BSR_ATTN_F16) {
        switch (c.D) {
            case 32: return fwd_two_pass_impl<_Float16, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_two_pass_impl<_Float16, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_two_pass_impl<_Float16, 128>(c, q, k, v, o, row_max, row_denom, ws);
            case 256: return fwd_two_pass_impl<_Float16, 256>(c, q, k, v, o, row_max, row_denom, ws);
            case 512: return fwd_two_pass_impl<_Float16, 512>(c, q, k, v, o, row_max, row_denom, ws);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.dtype == BSR_ATTN_BF16) {
        switch (c.D) {
            case 32: return fwd_two_pass_impl<__bf16, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_two_pass_impl<__bf16, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_two_pass_impl<__bf16, 128>(c, q, k, v, o, row_max, row_denom, ws);
            case 256: return fwd_two_pass_impl<__bf16, 256>(c, q, k, v, o, row_max, row_denom, ws);
            case 512: return fwd_two_pass_impl<__bf16, 512>(c, q, k, v, o, row_max, row_denom, ws);
        }
    } else {
        switch (c.D) {
            case 32: return fwd_two_pass_impl<float, 32>(c, q, k, v, o, row_max, row_denom, ws);
            case 64: return fwd_two_pass_impl<float, 64>(c, q, k, v, o, row_max, row_denom, ws);
            case 128: return fwd_two_pass_impl<float, 128>(c, q, k, v, o, row_max, row_denom, ws);
        }
    }
    return hipErrorInvalidValue;
}

int launch_bwd_at(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o,
                  const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                  void *ws) {
    if (c.dtype == BSR_ATTN_F16) {
        switch (c.D) {
            case 32: return bwd_impl<_Float16, 32>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 64: return bwd_impl<_Float16, 64>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 128: return bwd_impl<_Float16, 128>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 256: return bwd_impl<_Float16, 256>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 512: return bwd_wide_impl<_Float16>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            default: return hipErrorInvalidValue;
        }
    }
    if (c.dtype == BSR_ATTN_BF16) {
        switch (c.D) {
            case 32: return bwd_impl<__bf16, 32>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 64: return bwd_impl<__bf16, 64>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 128: return bwd_impl<__bf16, 128>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 256: return bwd_impl<__bf16, 256>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 512: return bwd_wide_impl<__bf16>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
        }
    } else {
        switch (c.D) {
            case 32: return bwd_impl<float, 32>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 64: return bwd_impl<float, 64>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 128: return bwd_impl<float, 128>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
        }
    }
    return hipErrorInvalidValue;
}

int launch_bwd_ds_at(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o,
                     const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                     void *ws) {
    if (c.dtype == BSR_ATTN_F16) {
        switch (c.D) {
            case 32: return bwd_ds_impl<_Float16, 32>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 64: return bwd_ds_impl<_Float16, 64>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 128: return bwd_ds_impl<_Float16, 128>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 256: return bwd_ds_impl<_Float16, 256>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 512: return bwd_wide_impl<_Float16>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
        }
    } else if (c.dtype == BSR_ATTN_BF16) {
        switch (c.D) {
            case 32: return bwd_ds_impl<__bf16, 32>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 64: return bwd_ds_impl<__bf16, 64>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 128: return bwd_ds_impl<__bf16, 128>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 256: return bwd_ds_impl<__bf16, 256>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
            case 512: return bwd_wide_impl<__bf16>(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
        }
    }
    return hipErrorInvalidValue;
}

// Copies up to five [BH*S, from] tensors to [BH*S, to] (zero-filled or cut).
int repack(const LaunchCommon &c, int n, const void *const *src, void *const *dst, int from, int to) {
    RepackArgs a{};
    for (int i = 0; i < n; ++i) {
        a.src[i] = static_cast<const int4 *>(src[i]);
        a.dst[i] = static_cast<int4 *>(dst[i]);
    }
    const int e = static_cast<int>(elem_bytes(c.dtype));
    a.rows = static_cast<int64_t>(c.BH) * c.S;
    a.src_chunks = from * e / 16;
    a.dst_chunks = to * e / 16;
    const int64_t total = a.rows * a.dst_chunks;
    const int blocks = static_cast<int>(std::min<int64_t>((total + NT - 1) / NT, 8 * compute_units()));
    if (blocks == 0) return 0;
    hipStream_t st = static_cast<hipStream_t>(c.stream);
    KernelTimer tm("repack", c.dtype == BSR_ATTN_F32 ? "fp32" : c.dtype == BSR_ATTN_BF16 ? "bf16" : "fp16", 0, st);
    hipLaunchKernelGGL(repack_kernel, dim3(blocks, n), dim3(NT), 0, st, a);
    return hipGetLastError();
}

// A head dim without an instance of its own: the operands are copied into
// zero-padded rows of the next instantiated width, the call runs there, and
// the outputs' real columns are copied back. Zero columns change no score
// (Q K^T sums over them as zeros) and produce zero columns in O, dQ, dK and
// dV (the padded V, K, Q and dO columns are zero), so the result equals the
// unpadded attention.
struct Padded {
    int Dp;
    char *base;
    size_t tensor;
    void *t(int i) const { return base + static_cast<size_t>(i) * tensor; }
};
Padded padded(const LaunchCommon &c, void *ws, int kind) {
    const int Dp = padded_head_dim(c.dtype, c.D);
    const size_t inst = instance_workspace(*c.s, c.BH, c.S, Dp, c.dtype, kind);
    const PadWorkspace pw = pad_workspace(inst, c.BH, c.S, c.D, c.dtype, kind ? kBwdPadTensors : kFwdPadTensors);
    return Padded{Dp, static_cast<char *>(ws) + pw.base, pw.tensor};
}

template <typename Launcher>
int forward_padded(Launcher launch, const LaunchCommon &c, const void *q, const void *k, const void *v, void *o,
                   float *row_max, float *row_denom, void *ws) {
    const Padded pd = padded(c, ws, 0);
    LaunchCommon cp = c;
    cp.D = pd.Dp;
    const void *in[3] = {q, k, v};
    void *inp[3] = {pd.t(0), pd.t(1), pd.t(2)};
    int err = repack(c, 3, in, inp, c.D, pd.Dp);
    if (err == 0) err = launch(cp, pd.t(0), pd.t(1), pd.t(2), pd.t(3), row_max, row_denom, ws);
    const void *out[1] = {pd.t(3)};
    void *outp[1] = {o};
    if (err == 0) err = repack(c, 1, out, outp, pd.Dp, c.D);
    return err;
}

template <typename Launcher>
int backward_padded(Launcher launch, int kind, const LaunchCommon &c, const void *q, const void *k, const void *v,
                    const void *o, const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk,
                    void *dv, void *ws) {
    if (native_head_dim(c.dtype, c.D)) return launch(c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
    const Padded pd = padded(c, ws, kind);
    LaunchCommon cp = c;
    cp.D = pd.Dp;
    const void *in[5] = {q, k, v, o, d_o};
    void *inp[5] = {pd.t(0), pd.t(1), pd.t(2), pd.t(3), pd.t(4)};
    int err = repack(c, 5, in, inp, c.D, pd.Dp);
    if (err == 0)
        err = launch(cp, pd.t(0), pd.t(1), pd.t(2), pd.t(3), pd.t(4), row_max, row_denom, pd.t(5), pd.t(6), pd.t(7),
                     ws);
    const void *out[3] = {pd.t(5), pd.t(6), pd.t(7)};
    void *outp[3] = {dq, dk, dv};
    if (err == 0) err = repack(c, 3, out, outp, pd.Dp, c.D);
    return err;
}

}  // namespace

int launch_fwd(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o, float *row_max,
               float *row_denom, void *ws) {
    if (native_head_dim(c.dtype, c.D)) return launch_fwd_at(c, q, k, v, o, row_max, row_denom, ws);
    return forward_padded(launch_fwd_at, c, q, k, v, o, row_max, row_denom, ws);
}

int launch_fwd_two_pass(const LaunchCommon &c, const void *q, const void *k, const void *v, void *o,
                        float *row_max, float *row_denom, void *ws) {
    if (native_head_dim(c.dtype, c.D)) return launch_fwd_two_pass_at(c, q, k, v, o, row_max, row_denom, ws);
    return forward_padded(launch_fwd_two_pass_at, c, q, k, v, o, row_max, row_denom, ws);
}

int launch_bwd(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o, const void *d_o,
               const float *row_max, const float *row_denom, void *dq, void *dk, void *dv, void *ws) {
    return backward_padded(launch_bwd_at, 1, c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
}

int launch_bwd_ds(const LaunchCommon &c, const void *q, const void *k, const void *v, const void *o,
                  const void *d_o, const float *row_max, const float *row_denom, void *dq, void *dk, void *dv,
                  void *ws) {
    return backward_padded(launch_bwd_ds_at, 2, c, q, k, v, o, d_o, row_max, row_denom, dq, dk, dv, ws);
}

int launch_mfma_probe(int dtype, int iters, float *sink, void *stream, double *flops) {
    const int blocks = 2 * compute_units();  // two workgroups (eight waves) per CU: two per SIMD
    hipStream_t st = static_cast<hipStream_t>(stream);
    const double per_mfma = dtype == BSR_ATTN_F32 ? 2.0 * 32 * 32 * 2 : 2.0 * 32 * 32 * 16;
    *flops = static_cast<double>(blocks) * (NT / 64) * 4.0 * iters * per_mfma;
    switch (dtype) {
        case BSR_ATTN_BF16: hipLaunchKernelGGL(mfma_probe_kernel<__bf16>, dim3(blocks), dim3(NT), 0, st, iters, sink); break;
        case BSR_ATTN_F16: hipLaunchKernelGGL(mfma_probe_kernel<_Float16>, dim3(blocks), dim3(NT), 0, st, iters, sink); break;
        case BSR_ATTN_F32: hipLaunchKernelGGL(mfma_probe_kernel<float>, dim3(blocks), dim3(NT), 0, st, iters, sink); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

int launch_spmm(const SpmmCommon &c, const void *blocks, const void *b, void *cm, void *ws) {
    switch (c.dtype) {
        case BSR_ATTN_F32: return spmm_impl<float>(c, blocks, b, cm, ws);
        case BSR_ATTN_BF16: return spmm_impl<__bf16>(c, blocks, b, cm, ws);
        case BSR_ATTN_F16: return spmm_impl<_Float16>(c, blocks, b, cm, ws);
        default: return hipErrorInvalidValue;
    }
}

const char *hip_error_string(int err) { return hipGetErrorString(static_cast<hipError_t>(err)); }

// Workspace of the no-allocation backward (bsr_attn_bwd_noalloc): a
// file-scope device array, one copy per GPU the library runs on, held until
// the process ends. Host code must not pass `scratch` itself to a kernel (on
// the host it names a stand-in, not the device copy): it uses the address
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept below.
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int scratch_pointer(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace bsr
