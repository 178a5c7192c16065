// Device-side helpers shared by the libfa355 kernels (gfx950 / CDNA4 only).
//
// Matrix-core conventions used throughout (one 64-lane wavefront; lane l,
// l32 = l % 32, hi = l / 32):
//
//   v_mfma_f32_32x32x16_{bf16,f16}:  D[32x32] += A[32x16] * B[16x32]
//     A operand: lane l holds A[l32][8*hi .. 8*hi+7]      (8 x 16-bit)
//     B operand: lane l holds B[8*hi .. 8*hi+7][l32]      (8 x 16-bit)
//     D / C    : lane l, register r holds D[row(r, hi)][l32] with
//                row(r, hi) = 8*(r/4) + 4*hi + (r%4)        (16 x fp32)
//   v_mfma_f32_32x32x2_f32:          D[32x32] += A[32x2] * B[2x32]
//     A: lane l holds A[l32][hi];  B: lane l holds B[hi][l32];  D as above.
//
// Both operands are contiguous along the contraction index inside a lane,
// which is what decides every LDS layout in the kernels.
#pragma once

#include <hip/hip_runtime.h>

#include "fa_launch.h"

#include <atomic>
#include <utility>
#include <stdint.h>

// Tile parameters of the default kernels.  A build may override them (-D) to
// produce an alternative library for measurements; the library the package
// ships and tests is built with these values.
#ifndef FA355_FWD_NW128
#define FA355_FWD_NW128 8      // forward waves per workgroup at d = 128
#endif
#ifndef FA355_FWD_BC128
#define FA355_FWD_BC128 64     // forward keys per tile at d = 128
#endif
#ifndef FA355_FWD_QLDS
#define FA355_FWD_QLDS 1       // forward persistent grid: Q and output staged in LDS
#endif
#ifndef FA355_FWD_PERSIST
#define FA355_FWD_PERSIST 1    // forward persistent grid
#endif
#ifndef FA355_FWD_STACK
#define FA355_FWD_STACK 1      // forward: stack the query heads of a K/V group
#endif
#ifndef FA355_DKDV_BQ128
#define FA355_DKDV_BQ128 128   // dK/dV query rows per step at d = 128
#endif
#ifndef FA355_DKDV_AHEAD
#define FA355_DKDV_AHEAD 4     // dK/dV operand read distance, in products
#endif
#ifndef FA355_DQ_NW
#define FA355_DQ_NW 4          // dQ waves per workgroup
#endif
#ifndef FA355_SPLIT_NS
#define FA355_SPLIT_NS 2       // LDS stages of the split-KV chunk kernel
#endif
#ifndef FA355_DQ_BC128
#define FA355_DQ_BC128 64      // dQ keys per tile at d = 128
#endif

// Clock probe, for measurement builds only (-DFA355_CLOCK_PROBE=1).  Each wave of
// the forward, dK/dV and dQ kernels records the shader-clock counter and the
// fixed 100 MHz real-time counter when it starts and when it ends, one record
// per wave slot (blockIdx.x * waves + wave, the first FA355_CLOCK_PROBE_SLOTS
// slots), read back by <array>_read(host).  Their ratio is the clock the chip
// ran the kernel at; the spread of the end times is the grid's tail.  The
// default library compiles all of it away.
#ifndef FA355_CLOCK_PROBE
#define FA355_CLOCK_PROBE 0
#endif
#if FA355_CLOCK_PROBE
#define FA355_CLOCK_PROBE_SLOTS 8192
#define FA355_CLOCK_PROBE_ARRAY(NAME)                                                      \
    __device__ unsigned long long NAME[FA355_CLOCK_PROBE_SLOTS][4];                         \
    extern "C" int NAME##_read(void* host) {                                               \
        return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(NAME), sizeof(NAME), 0,            \
                                        hipMemcpyDeviceToHost);                            \
    }
#define FA355_CLOCK_BEGIN                                                                  \
    const unsigned long long clock_c0_ = __builtin_amdgcn_s_memtime();                     \
    const unsigned long long clock_r0_ = __builtin_amdgcn_s_memrealtime();
#define FA355_CLOCK_END(NAME)                                                              \
    {                                                                                     \
        const unsigned long long c1 = __builtin_amdgcn_s_memtime();                        \
        const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();                    \
        const unsigned slot = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;           \
        if ((threadIdx.x & 63) == 0 && slot < FA355_CLOCK_PROBE_SLOTS) {                   \
            unsigned long long* rec = NAME[slot];                                          \
            rec[0] = clock_c0_;                                                            \
            rec[1] = c1;                                                                   \
            rec[2] = clock_r0_;                                                            \
            rec[3] = r1;                                                                   \
        }                                                                                 \
    }
#else
#define FA355_CLOCK_PROBE_ARRAY(NAME)
#define FA355_CLOCK_BEGIN
#define FA355_CLOCK_END(NAME)
#endif

namespace fa355 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element-type tags for the 16-bit paths.
struct BF16 {};
struct FP16 {};

template <typename T>
struct Mma;

template <>
struct Mma<BF16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    // Two fp32 values -> one dword of two round-to-nearest-even bf16 values.
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        bf16x2 r;
        r[0] = (__bf16)lo;
        r[1] = (__bf16)hi;
        return __builtin_bit_cast(uint32_t, r);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return __uint_as_float(((uint32_t)x) << 16);
    }
};

template <>
struct Mma<FP16> {
    static __device__ __forceinline__ f32x16 mma(u32x4 a, u32x4 b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    static __device__ __forceinline__ uint32_t pack2(float lo, float hi) {
        f16x2 r;
        r[0] = (_Float16)lo;
        r[1] = (_Float16)hi;
        return __builtin_bit_cast(uint32_t, r);
    }
    static __device__ __forceinline__ float to_f32(uint16_t x) {
        return (float)__builtin_bit_cast(_Float16, x);
    }
};

__device__ __forceinline__ f32x16 mma_f32(float a, float b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x16 zero16() {
    f32x16 z;
#pragma unroll
    for (int i = 0; i < 16; ++i) z[i] = 0.f;
    return z;
}

// Row (within a 32x32 accumulator block) held by register r of a lane in
// half `hi` of the wave.
__device__ __forceinline__ constexpr int acc_row(int r, int hi) {
    return 8 * (r >> 2) + 4 * hi + (r & 3);
}

// Value of lane (l ^ 32): exchange between the two halves of the wave.
__device__ __forceinline__ float swap_halves(float x) {
    return __shfl_xor(x, 32, 64);
}

// max(x[l], x[l ^ 32]) for every lane l, on the vector unit: one
// v_permlane32_swap exchanges the upper half of one copy with the lower half
// of the other, so the two results hold both values of each lane pair.
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Lazy rescale threshold of the online softmax (log2 units): the running
// maximum moves only when a tile's maximum exceeds it by more than this, so
// unnormalised probabilities stay below 2^kTau and the result stays exact
// (the output and the row sum always refer to the same maximum).
constexpr float kTau = 8.0f;

// Native 2^x (v_exp_f32); exp2(-inf) = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are handed to the 8 XCDs of the chip round-robin, and each XCD
// has its own L2.  Renumber so that XCD x runs a contiguous range of logical
// blocks: neighbouring logical blocks (same head, same K/V) then share an L2.
__device__ __forceinline__ int xcd_remap(int pid, int total) {
    constexpr int kXcd = 8;
    const int xcd = pid % kXcd;
    const int local = pid / kXcd;
    const int per = total / kXcd;
    const int rem = total % kXcd;
    return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// Persistent schedule: XCD x = p % 8 owns the logical blocks that xcd_remap
// gives it; its G / 8 workgroups (G a multiple of 8), i = p / 8, take the
// range's k-th block in round r for k = r G/8 + (r even ? i : G/8 - 1 - i),
// a snake that pairs long and short rows over consecutive rounds.  -1 once
// the range is exhausted (k only grows with r).
__device__ __forceinline__ int persist_block(int p, int G, int total, int round) {
    constexpr int kXcd = 8;
    const int x = p % kXcd, i = p / kXcd, gx = G / kXcd;
    const int per = total / kXcd, rem = total % kXcd;
    const int cnt = per + (x < rem ? 1 : 0);
    const int start = x < rem ? x * (per + 1) : rem * (per + 1) + (x - rem) * per;
    const int k = round * gx + ((round & 1) ? gx - 1 - i : i);
    return k < cnt ? start + k : -1;
}

// The shared tail of that schedule: once every workgroup has walked its first
// rs rounds (stat = rs * G/8 blocks of each XCD's range), the blocks left in
// XCD y's range form its pool, ordered longest first where the pool is whole
// heads of nqb row (or key) blocks (position c is block c / heads of head
// c % heads; under the causal mask the logical numbering puts a head's longest
// block first).  pool[y] packs two counters: the low 16 bits count claims from
// the front, the high 16 from the back.  A workgroup on XCD x takes pool x's
// front (the longest block left, its heads in its own L2); once that pool is
// empty it takes the back (the shortest block left) of x + 1, x + 2, ...  A
// claim is valid while front + back < the pool's size, so no position is
// handed out twice.  A workgroup that finds every pool empty counts itself in
// pool[8]; the last of the grid resets the counters for the next launch that
// takes this slot.  Returns the block, or -1.  (The caller keeps the schedule
// static where a counter could pass 16 bits.)
__device__ __forceinline__ int claim_pooled(unsigned* pool, int x, int total, int stat, int nqb,
                                            unsigned grid) {
    constexpr int kXcd = 8;
    const int per = total / kXcd, rem = total % kXcd;
    for (int t = 0; t < kXcd; ++t) {
        const int y = (x + t) % kXcd;
        const int rest = (y < rem ? per + 1 : per) - stat;
        if (rest <= 0) continue;
        const unsigned old = atomicAdd(&pool[y], t == 0 ? 1u : 0x10000u);
        const int f = (int)(old & 0xffffu), bk = (int)(old >> 16);
        if (f + bk < rest) {
            const int c = t == 0 ? f : rest - 1 - bk;
            const int start = y < rem ? y * (per + 1) : rem * (per + 1) + (y - rem) * per;
            const int lo = start + stat;
            if (lo % nqb == 0 && rest % nqb == 0) {
                const int heads = rest / nqb;
                return lo + (c % heads) * nqb + c / heads;
            }
            return lo + c;
        }
    }
    if (atomicAdd(&pool[kXcd], 1u) == grid - 1)
        for (int y = 0; y <= kXcd; ++y) atomicExch(&pool[y], 0u);
    return -1;
}

// Workgroups in a persistent grid of one workgroup per compute unit of the
// current device, rounded down to a multiple of the 8 XCDs (0 if unknown).
// The compute-unit count is cached per device in relaxed atomics: threads that
// race on a first call each query the device and store the same value.
inline int persistent_grid() {
    static std::atomic<int> cus[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int c = cus[dev].load(std::memory_order_relaxed);
    if (c == 0) {
        int n = 0;
        c = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0 ? n : -1;
        cus[dev].store(c, std::memory_order_relaxed);
    }
    return c > 0 ? c / 8 * 8 : 0;
}

// Raw buffer resource over one tensor region of `bytes` bytes.  Loads whose
// byte offset lies at or past `bytes` return zeros (hardware range check), so
// rows past the end of a sequence need no branch.  The offset is always passed
// in the per-lane operand, which the range check covers.
struct Buf {
    __amdgpu_buffer_rsrc_t r;
    __device__ __forceinline__ Buf(const void* base, uint32_t bytes)
        : r(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000)) {}
    __device__ __forceinline__ u32x4 load16(uint32_t off) const {
        return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    }
    __device__ __forceinline__ float load_f32(uint32_t off) const {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, 0));
    }
};

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Asynchronous copy of 16 bytes per lane from a buffer (byte offset `off`,
// zeros past the range) into LDS at `lds + 16 * lane`; `lds` must be
// wave-uniform.  Completion is tracked by the vector-memory counter.
__device__ __forceinline__ void buf_to_lds16(const Buf& b, void* lds, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(b.r, (lds_ptr_t)lds, 16, (int)off, 0, 0, 0);
}

// Wait until this wave's outstanding vector-memory operations (including
// buffer-to-LDS copies) have completed.
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's vector-memory operations are
// outstanding (they complete in issue order, so the older ones are done).
template <int N>
__device__ __forceinline__ void wait_vmem_n() {
    static_assert(N >= 0 && N <= 63, "vmcnt holds 6 bits");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Transposing LDS read (ds_read_b64_tr_b16).  Within each group of 16 lanes,
// lane i receives element (i % 4) of the 8-byte chunk addressed by lane
// 4*k + i/4, for k = 0..3: when lane s addresses row r0 + s/4, columns
// c0 + 4*(s % 4) .. +3 of a row-major 16-bit tile, lane i gets
// column c0 + i of rows r0 .. r0 + 3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 ld_global16(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ u32x4 zero_u4() {
    u32x4 z;
    z[0] = z[1] = z[2] = z[3] = 0u;
    return z;
}

// Row-major tile in LDS (row = key or query, D 16-bit elements): 16-byte chunk
// c of row r is stored at chunk c ^ (r & 7) so that the 32 lanes reading one chunk column of
// 32 consecutive rows spread over all banks.
template <int D>
__device__ __forceinline__ int k_off(int row, int chunk) {
    return row * (D * 2) + ((chunk ^ (row & 7)) << 4);
}

// Transposed tile in LDS (row = head-dim index, BC 16-bit elements in
// "position" order, see v_key_of_pos), chunk c of row r stored at
// c ^ ((r ^ (r >> 3)) & 7): conflict-free both for the transposing writes
// (rows 8 apart) and for the operand reads (consecutive rows).
template <int BC>
__device__ __forceinline__ int v_off(int row, int chunk) {
    return row * (BC * 2) + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

// LDS on gfx950 serves a 128-bit read for 16 lanes per cycle across 64 banks
// (256 bytes), and a 64-bit read for 32 lanes.  The layouts below keep every
// such group of lanes on distinct banks (and also every 8-lane group within a
// 128-byte window).
//
// Row-major tile read as an MFMA A operand (lane l32 reads row l32, one
// 16-byte chunk): chunk c of row r is stored at c ^ (r & 15) for 16 chunks
// per row, c ^ ((r ^ (r >> 3)) & 7) for 8.
template <int D>
__device__ __forceinline__ int kq_off(int row, int chunk) {
    const int sw = (D == 128) ? (row & 15) : ((row ^ (row >> 3)) & 7);
    return row * (D * 2) + ((chunk ^ sw) << 4);
}

// Row-major tile read with the transposing read (four rows of 32 bytes per
// 16-lane group, 64 bytes per 32-lane group): chunk c of row r is stored at
// c ^ s(r & 3) with s = {0, 6, 12, 10} for 16 chunks per row (distinct in
// chunk bits 1-2 and 2-3), s = {0, 2, 4, 6} for 8.
template <int D>
__device__ __forceinline__ int tr_swz(int row) {
    if (D == 128) return ((row & 1) * 6) ^ (((row >> 1) & 1) * 12);
    return 2 * (row & 3);
}
template <int D>
__device__ __forceinline__ int vt_off(int row, int byte_in_row) {
    return row * (D * 2) + ((((byte_in_row >> 4) ^ tr_swz<D>(row)) << 4) | (byte_in_row & 15));
}

// Row-major tile read both ways: as MFMA A operands (16 consecutive rows per
// 128-bit read) and through the transposing read (4-row groups).  Chunk c of
// row r is stored at c ^ sw(r) with sw(r) = f[r & 3] ^ ((r >> 2) & 3),
// f = {0, 4, 10, 14} for 16 chunks per row and {0, 2, 4, 6} for 8: distinct
// for 16 consecutive rows, and within each aligned 4-row group distinct in
// chunk bits 1-2 and 2-3 (64-bank and 32-bank conflict-free for both reads).
// An LDS byte offset made opaque to the optimiser (so that it stays in one
// register instead of being re-derived at every use) and then bounded, so the
// constant parts of later addresses still fold into the instruction offset.
__device__ __forceinline__ uint32_t lds_lane_off(uint32_t x) {
    asm volatile("" : "+v"(x));
    return x & 0x3FFFFu;
}

// Compile-time loop: calls f(std::integral_constant<int, i>) for i = 0..N-1,
// so every index inside f is a constant expression (unrolling guaranteed).
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>) {
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

template <int D>
__device__ __forceinline__ int dual_swz(int row) {
    const int r3 = row & 3;
    const int f = (D == 128) ? ((r3 & 1) * 4 + (r3 >> 1) * 10) : 2 * r3;
    return f ^ ((row >> 2) & 3);
}
template <int D>
__device__ __forceinline__ int dual_off(int row, int byte_in_row) {
    return row * (D * 2) + ((((byte_in_row >> 4) ^ dual_swz<D>(row)) << 4) | (byte_in_row & 15));
}

// Inside a 16-element group of a transposed tile, elements are stored in the
// order in which a 32x32 accumulator hands them to the next product as its B
// operand: position 8*h + i (h = lane half, i = 0..7) holds element
// 4*h + (i & 3) + 8*(i >> 2) of the group.
__device__ __forceinline__ int v_key_of_pos(int h, int i) { return 4 * h + (i & 3) + 8 * (i >> 2); }

// Inverse: position of element x (0..15) of a group.
__device__ __forceinline__ int pos_of_elem(int x) {
    return 8 * ((x >> 2) & 1) + 4 * ((x >> 3) & 1) + (x & 3);
}

// ---------------------------------------------------------------- dropout
//
// Keep mask of attention dropout.  Element (b, h, i, j) (query head h, row i,
// key j) is kept iff its random byte is below t8 = round((1 - p) 256); kept
// probabilities are scaled by 256 / t8.  The bytes come from the
// counter-based generator Philox4x64-10 (Salmon, Moraes, Dror and Shaw,
// "Parallel random numbers: as easy as 1, 2, 3", SC 2011) with key
// (seed, offset) and counter (j / 32, i, b H_q + h, 0): one call gives the
// 32 bytes of one row and one aligned 32-key block, little-endian, byte
// j % 32 for key j (dword (j % 32) / 4 of the result).
// Philox4x64 state, advanced one round at a time, so that a kernel can spread
// the ten rounds over instructions that would otherwise wait.
struct Philox4x64 {
    uint64_t c[4];
    uint64_t k0, k1;
    // counter (kblk, row, bh, 0), key (seed, offset)
    __device__ __forceinline__ void start(uint32_t kblk, uint32_t row, uint32_t bh, const DropParams& dp) {
        c[0] = kblk;
        c[1] = row;
        c[2] = bh;
        c[3] = 0;
        k0 = dp.seed;
        k1 = dp.offset;
    }
    __device__ __forceinline__ void round() {
        // multipliers and Weyl key increments of Philox4x64 (Salmon et al.)
        constexpr uint64_t M0 = 0xD2E7470EE14C6C93ull, M1 = 0xCA5A826395121157ull;
        constexpr uint64_t W0 = 0x9E3779B97F4A7C15ull, W1 = 0xBB67AE8584CAA73Bull;
        const uint64_t lo0 = M0 * c[0], hi0 = __umul64hi(M0, c[0]);
        const uint64_t lo1 = M1 * c[2], hi1 = __umul64hi(M1, c[2]);
        const uint64_t n0 = hi1 ^ c[1] ^ k0;
        const uint64_t n2 = hi0 ^ c[3] ^ k1;
        c[0] = n0;
        c[1] = lo1;
        c[2] = n2;
        c[3] = lo0;
        k0 += W0;
        k1 += W1;
    }
    // the 32 output bytes as 8 little-endian dwords
    __device__ __forceinline__ void words(uint32_t w[8]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            w[2 * i] = (uint32_t)c[i];
            w[2 * i + 1] = (uint32_t)(c[i] >> 32);
        }
    }
};

// The 32 random bytes of (row, key block kblk) of head index bh, as 8 dwords.
__device__ __forceinline__ void drop_bytes(uint32_t w[8], uint32_t kblk, uint32_t row, uint32_t bh,
                                           const DropParams& dp) {
    Philox4x64 g;
    g.start(kblk, row, bh, dp);
#pragma unroll
    for (int r = 0; r < 10; ++r) g.round();
    g.words(w);
}

// In the score layouts where a lane owns one query row and, in each 32-key
// block, keys 8 g + 4 hi + (0..3) for g = 0..3 (register 4 g + i), a lane
// needs dword 2 g + hi of that block's bytes.  When lane half hi has
// computed the bytes w of block (pair base + hi), one v_permlane32_swap per g
// hands every lane its dwords of both blocks of the pair: m0 for the first,
// m1 for the second.
__device__ __forceinline__ void drop_pair_exchange(const uint32_t w[8], uint32_t m0[4], uint32_t m1[4]) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
        const auto r = __builtin_amdgcn_permlane32_swap(w[2 * g], w[2 * g + 1], false, false);
        m0[g] = r[0];
        m1[g] = r[1];
    }
}

// Byte i of dword m kept?
__device__ __forceinline__ bool drop_keep(uint32_t m, int i, int t8) {
    return (int)((m >> (8 * i)) & 0xFFu) < t8;
}

typedef short s16x2 __attribute__((ext_vector_type(2)));

// Mask for a dword of two 16-bit values built from bytes i0 and i0 + 1 of m:
// 0xFFFF in each half whose byte is below t8, else 0.
__device__ __forceinline__ uint32_t drop_mask16x2(uint32_t m, int i0, int t8) {
    const uint32_t sel = (uint32_t)i0 | (0x0Cu << 8) | ((uint32_t)(i0 + 1) << 16) | (0x0Cu << 24);
    const uint32_t x = __builtin_amdgcn_perm(0u, m, sel);   // bytes -> 16-bit halves
    s16x2 v = __builtin_bit_cast(s16x2, x);
    const s16x2 t = {(short)t8, (short)t8};
    v = (v - t) >> (short)15;
    return __builtin_bit_cast(uint32_t, v);
}

}  // namespace fa355
