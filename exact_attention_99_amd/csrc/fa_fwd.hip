// Forward pass of exact tiled attention with online softmax, gfx950.
//
// One workgroup owns BR = 32 * NW query rows of one (batch, query head); each
// of its NW waves owns 32 of them.  The workgroup walks the key/value tiles of
// BC keys in ascending order (causal: only up to its last row), staging each
// tile in LDS while the previous one is being used ("FlashAttention and the
// Kernel Era", The Breakthrough: load one block of each of Q, K, V into fast
// on-chip memory and fold the partial result into a running output).
//
// Per tile a wave computes S^T = K Q^T on the matrix cores, so that lane l
// owns query row l % 32 and holds 16 of its scores per 32-key block; the row
// maximum is then an in-lane reduction plus one exchange between the two
// halves of the wave.  The running maximum m and running sum l follow the
// online-softmax update ("FlashAttention and the Kernel Era", The Mathematics,
// online-softmax equation; "FlashAttention 1, 2, and 3 Explained", section 2:
// rescale the accumulated output by e^(m_old - m_new)).  P~^T stays in
// registers and is directly the B operand of O^T += V^T P~^T.  The output is
// divided by l once at the end and the natural-log logsumexp is written for
// the backward pass.
//
// Exponentials are taken base 2 with scale * log2(e) folded into one FMA.
// The running maximum is only moved when a tile's maximum exceeds it by more
// than kTau (in log2 units): the skipped rescales leave every result exact,
// because O and l always refer to the same m, and P~ stays below 2^kTau.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa355 {

FA355_CLOCK_PROBE_ARRAY(fa355_clock_fwd)

// Counters of the persistent forward's shared tail: a ring of 64-byte slots
// (a claim counter per XCD and a done counter each), one slot per launch,
// chosen round-robin on the host.  A launch leaves its slot at zero when it ends, so
// launches that overlap in time (other streams) stay apart as long as fewer
// than kPoolSlots of them are in flight on one device at once.
constexpr int kPoolSlots = 64;
__device__ __attribute__((aligned(64))) unsigned fa355_fwd_pool[kPoolSlots * 16];

// This launch's slot on the current device (nullptr if the symbol's address
// cannot be had: the kernel then keeps its static schedule).
unsigned* fwd_pool_slot() {
    static std::atomic<unsigned*> base[64];
    static std::atomic<unsigned> seq{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    unsigned* p = base[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(fa355_fwd_pool)) != hipSuccess || !a) return nullptr;
        p = static_cast<unsigned*>(a);
        base[dev].store(p, std::memory_order_release);
    }
    return p + 16 * (seq.fetch_add(1, std::memory_order_relaxed) % kPoolSlots);
}

namespace {

// Sixth-generation 16-bit forward kernel: NW waves of 32 query rows, tiles of
// 64 keys.
//
// Data path.  K and V tiles go from global memory straight into LDS by
// buffer-to-LDS copies (no staging registers; rows past the end of the
// sequence arrive as zeros), both row-major, double-buffered: the copy of tile
// j + 1 is issued at the start of tile j.  The V^T operand of the P V product
// comes from transposing LDS reads.  Tiles that lie wholly at or below every
// row of the block and inside the sequence run a body with no mask code, two
// at a time so that both LDS buffers are compile-time constants; the diagonal
// and ragged-end tiles run the masked body, and a wave skips tiles above its
// rows.  A tile's LDS reads go through a restrict-qualified pointer to its
// buffer, so the compiler does not make them wait for the copies of the next
// tile into the other buffer.
//
// Softmax.
// 1. The running maximum is not recomputed per tile.  The probabilities of a
//    32-key half tile are formed against the current maximum m and summed; if
//    every lane's sum stays at or below 2^kTau (and m is finite), no
//    probability exceeds 2^kTau either, so the unnormalised values are in
//    range and the half is accepted as it is: the output and the row sum still
//    refer to the same m, and the result is exact.  Otherwise (the first tile
//    of a row, or scores that rose above m) the wave takes the slow path: the
//    half's true row maximum, the rescale of the output and row sum, and the
//    probabilities again.
// 2. The two halves of a tile are pipelined inside the wave: the scores of
//    the second half are formed on the matrix cores while the vector unit
//    exponentiates the first, and the P V products of the first half run
//    while the second is exponentiated.
//
// PERSIST: the grid holds as many workgroups as fit on the device at once,
// and each walks the row blocks persist_block() assigns it, which saves a
// workgroup launch per block.  On this path (dense) Q also goes through LDS:
// each wave owns 32 rows of an LDS Q tile, copies the next block's Q rows
// there after writing its output, and stages its output rows there so that
// they leave in 1 KB stores of consecutive rows.
//
// DROP: attention dropout (fa_common.h) on the probabilities before the P V
// product; the row sums and lse stay those of the undropped probabilities.
// Lane half hi draws the bytes of key block k0 / 32 + hi of its row, and one
// exchange between the halves gives each lane its bytes of both blocks.
//
// SPARSE: block-sparse attention and variable-length batches (SparseParams).
// With a block mask the workgroup walks only the key tiles that the mask
// allows for one of its rows (the copy of the next such tile overlaps the
// current one), and a wave computes a tile only if its own 32 rows may see it;
// with sequence lengths the length replaces N in every range check.  Rows that
// see no key get O = 0 and lse = -inf.
template <typename T, int D, bool CAUSAL, int NW, int BC, bool PERSIST = false, bool DROP = false,
          bool SPARSE = false, int GS = 1>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
fwd16v6_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
               const uint16_t* __restrict__ V, uint16_t* __restrict__ O, float* __restrict__ LSE,
               int B, int Hq, int Hkv, int N, float cl2, DropParams dp, SparseParams sp,
               unsigned* __restrict__ pool) {
    FA355_CLOCK_BEGIN
    static_assert(BC == 64 || BC == 128, "tiles of one or two 64-key sub-tiles");
    static_assert(D == 64 || D == 128, "head dimensions with a K tile swizzle");
    constexpr int PPB = 8 / (D / 16);    // probability pairs per second-half score product
    constexpr int PPC = 8 / (2 * (D / 32));  // probability pairs per first-half P V product
    constexpr int NSUB = BC / 64;
    constexpr int BR = 32 * NW / GS;     // rows of each of the block's GS query heads
    constexpr int KCH = D / 8;
    constexpr int TILE = BC * D * 2;
    constexpr int STAGE = 2 * TILE;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr int WI = TILE / 1024;
    static_assert(WI % NW == 0, "tile copies split evenly over the waves");
    constexpr int IPW = WI / NW;
    static_assert(BR % BC == 0, "row blocks start on a key-tile boundary");
    // QL (the persistent dense path): Q goes through LDS as well, and the next
    // block's data is in flight before the current block ends.  Every wave
    // reads its Q fragments from its own 32 rows of an LDS Q tile (stored with
    // the K tiles' swizzle, so the reads are conflict-free) instead of issuing
    // 16-byte loads 256 bytes apart from global memory at the start of every
    // block, which cost several tile-times per block; right after those reads
    // it copies the next block's Q rows there.  The copy slot of the block's
    // last tile carries the next block's first K/V tile, so tile j of a block
    // lies in buffer (j + p0) & 1 with p0 alternating between blocks.  The
    // output rows are staged in LDS (the last tile's buffer and a spare
    // region) and leave in 1 KB stores of consecutive rows.
    // (d = 128 only, and only where the LDS still fits the 8 / NW workgroups per
    // compute unit that give 2 waves per SIMD; the d = 64 build runs 3 waves
    // per SIMD, which the larger LDS area and the extra registers would cost)
    constexpr bool QL = FA355_FWD_QLDS && PERSIST && !DROP && !SPARSE && D == 128 &&
                        (2 * STAGE + 48 * NW * D * 2) * (8 / NW) <= 160 * 1024;
    // QN (one row block per workgroup, 8 waves, d = 128: the dropout and
    // variable-length builds): the same Q tile, without the next block's
    // copies; each wave stages its output rows in its own Q rows.
    constexpr bool QN = FA355_FWD_QLDS && !PERSIST && D == 128 && NW == 8 && GS == 1 &&
                        2 * STAGE + 32 * NW * D * 2 <= 160 * 1024;
    // QB (the other builds whose Q rows fit one K/V buffer: 4 waves, at d = 64
    // or with a block mask): the same, with the Q rows in K/V buffer 1 before
    // the first tile (a second barrier keeps the first copy into that buffer
    // from overwriting them), so the LDS per workgroup stays as it is.  On the
    // persistent grid a wave that starts the next block early only copies into
    // its own rows of buffer 1 and into buffer 0, which every wave is done with.
    constexpr bool QB = FA355_FWD_QLDS && !QL && !QN && GS == 1 && 32 * NW * D * 2 <= STAGE;
    constexpr int QTILE = (QL || QN) ? 32 * NW * D * 2 : 0;
    constexpr int OSPARE = QL ? QTILE / 2 : 0;   // output staging of waves NW/2 .. NW - 1
    constexpr int OWAVE = 32 * D * 2;   // a wave's output rows
    static_assert(GS == 1 || (!DROP && !SPARSE && NW % GS == 0), "stacked query heads: dense path only");
    constexpr float kSumCap = 256.0f;   // 2^kTau
    static_assert(kTau == 8.0f, "sum cap matches the lazy-rescale threshold");

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE + QTILE + OSPARE];
    unsigned char* const qlds = smem + (QB ? STAGE : 2 * STAGE);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int nqb = (N + BR - 1) / BR;
    const int total = nqb * (Hq / GS) * B;

    // this lane's parts of the K/V tile copies (source offsets for its LDS
    // slots: chunk pc of row `row` holds the row's chunk pc ^ swizzle)
    uint32_t cpk[IPW], cpv[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int p = (wave + NW * i) * 64 + lane;
        const int row = p / KCH, pc = p % KCH;
        cpk[i] = (uint32_t)kq_off<D>(row, pc);
        cpv[i] = (uint32_t)(row * D * 2 + 16 * (pc ^ tr_swz<D>(row)));
    }
    // QL: block lg's coordinates; the copies of this wave's 32 Q rows into its
    // own 8 KB (d = 128) of the Q tile (rows ra0 .. ra0 + 31 of the tile, which
    // are rows q0 + 32 slice .. of head h0 + wave % GS), and this wave's share
    // of the copies of the block's first K/V tile into the buffer at `base`.
    // Rows past N read zeros (past the end of a head's range).
    // (The lane index is passed through an empty asm at each call, so that the
    // lane-dependent offsets are formed where the copies are issued instead of
    // being hoisted out of the block loop and held through every tile.)
    constexpr int QRPC = 1024 / (D * 2);   // Q rows per 1 KB copy
    const int slice_w = GS > 1 ? wave / GS : (wave < NW / 2 ? wave : (NW - 1) - (wave - NW / 2));
    const int ra0 = (GS > 1 ? (wave % GS) * BR : 0) + 32 * slice_w;
    unsigned char* const qown = qlds + ra0 * D * 2;
    auto block_of = [&](int lg, int& q00, int& h0, int& bb) {
        const int qbr = lg % nqb, bhh = lg / nqb;
        q00 = (CAUSAL ? (nqb - 1 - qbr) : qbr) * BR;
        h0 = GS > 1 ? (bhh % (Hq / GS)) * GS : bhh % Hq;
        bb = bhh / (Hq / GS);
    };
    auto issue_q = [&](int lg) {
        int ln = lane;
        asm volatile("" : "+v"(ln));
        int q00, h0, bb;
        block_of(lg, q00, h0, bb);
        const int hw = h0 + (GS > 1 ? wave % GS : 0);
        const Buf Qg(Q + ((size_t)bb * Hq + hw) * (size_t)N * D, (uint32_t)N * D * 2);
#pragma unroll
        for (int k = 0; k < 32 / QRPC; ++k) {
            const int r = QRPC * k + ln / KCH, pc = ln % KCH;   // local row, LDS chunk
            const uint32_t src = (uint32_t)(q00 + 32 * slice_w + r) * (D * 2);
            buf_to_lds16(Qg, qown + 1024 * k, src + (uint32_t)(kq_off<D>(ra0 + r, pc) - (ra0 + r) * D * 2));
        }
    };
    auto issue_kv0 = [&](int lg, unsigned char* base) {
        int q00, h0, bb;
        block_of(lg, q00, h0, bb);
        const size_t kv0 = ((size_t)bb * Hkv + h0 / (Hq / Hkv)) * (size_t)N * D;
        const Buf Kg(K + kv0, (uint32_t)N * D * 2), Vg(V + kv0, (uint32_t)N * D * 2);
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int bi = wave + NW * i;
            buf_to_lds16(Kg, base + bi * 1024, cpk[i]);
            buf_to_lds16(Vg, base + TILE + bi * 1024, cpv[i]);
        }
    };
    int p0 = 0;   // QL: buffer of the current block's tile 0
    // Shared tail (QL, with a pool slot): the XCDs of the chip run at clocks
    // that differ by up to ~10% under this kernel, so equal static shares end
    // when the slowest XCD does.  Every workgroup walks its first rs rounds of
    // persist_block statically; the blocks past them in each XCD's range (at
    // least two rounds' worth, an eighth of the work on long walks) are
    // claimed one at a time (claim_pooled: the workgroup's own XCD's pool
    // first, then the others'), so a faster XCD takes more of them.  Without a
    // slot every round is static, and so is every round without the causal
    // mask: its blocks are all as long as the longest causal ones, too coarse
    // to even out the XCDs' ends.
    constexpr bool TAIL = QL && CAUSAL;
    const int gxd = (int)gridDim.x / 8;
    const int rounds_x = gxd > 0 ? (total / 8) / gxd : 0;
    const int tail_rounds = max(2, rounds_x / 8);
    // (the 16-bit pool counters: each pool holds at most (tail_rounds + 1) G/8
    // blocks, its back counter counts at most all pooled claims and one failed
    // claim per workgroup)
    const bool fits16 = 9 * (tail_rounds + 1) * gxd + (int)gridDim.x < (1 << 16);
    const int rs = (TAIL && pool && fits16) ? max(0, rounds_x - tail_rounds) : 0x7fffffff;
    // One block per workgroup, or (PERSIST) a grid of one workgroup per compute
    // unit that walks its blocks in rounds.
    for (int round = 0;; ++round) {
        int logical, nxt = -1;
        bool fresh = round == 0;   // QL: nothing of this block is in flight yet
        if constexpr (PERSIST) {
            if (round < rs) {
                logical = persist_block((int)blockIdx.x, (int)gridDim.x, total, round);
                if (logical < 0) break;
                nxt = round + 1 < rs ? persist_block((int)blockIdx.x, (int)gridDim.x, total, round + 1) : -1;
            } else {
                if constexpr (TAIL) {
                    // the word goes through the spare staging region, which the
                    // previous block's epilogue is done with after this barrier
                    // and this block's epilogue writes only after later ones
                    int* const word = reinterpret_cast<int*>(smem + 2 * STAGE + QTILE);
                    __syncthreads();
                    if (tid == 0)
                        *word = claim_pooled(pool, (int)blockIdx.x % 8, total, rs * gxd, nqb, gridDim.x);
                    __syncthreads();
                    logical = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(word));
                    if (logical < 0) break;
                    fresh = true;
                    p0 = 0;
                } else {
                    break;
                }
            }
        } else {
            if (round > 0) break;
            logical = xcd_remap((int)blockIdx.x, total);
        }
        const int qb_raw = logical % nqb;
        const int bh = logical / nqb;
        const int qb = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;  // longest rows first
        // the masked path takes the batch index fastest, so that the XCDs (each
        // runs a contiguous range of heads) share sequences of different lengths.
        // GS > 1: the block is the same rows of GS query heads of one K/V group
        // (wave w serves head w % GS), which share every K/V tile.
        const int h = SPARSE ? bh / B : (GS > 1 ? (bh % (Hq / GS)) * GS + wave % GS : bh % Hq);
        const int b = SPARSE ? bh % B : bh / (Hq / GS);
        const int hk = h / (Hq / Hkv);

        const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
        const size_t koff = ((size_t)b * Hkv + hk) * (size_t)N * D;
        // valid positions of this sequence (variable lengths; else N).  Positions
        // past Nk read as zeros: padded queries then score 0 against every key,
        // and padded keys are masked.
        const int Nk = (SPARSE && sp.seqlens) ? min(max(sp.seqlens[b], 0), N) : N;
        const uint32_t head_bytes = (uint32_t)Nk * D * 2;
        const Buf Qb(Q + qoff, head_bytes), Kb(K + koff, head_bytes), Vb(V + koff, head_bytes);

        const int q0 = qb * BR;
        // waves w and w + NW/2 share a SIMD: give them complementary row slices
        // (w and NW - 1 - (w - NW/2)) so the diagonal tiles split evenly (with
        // stacked heads, wave w takes slice w / GS of its head)
        const int slice = GS > 1 ? wave / GS : (wave < NW / 2 ? wave : (NW - 1) - (wave - NW / 2));
        const int qw = q0 + 32 * slice;
        const int q = qw + l32;

        u32x4 qf[NKS];
        if constexpr (QL) {
            // the first block's copies are issued here, the others' during the
            // previous block
            if (fresh) {
                issue_q(logical);
                issue_kv0(logical, smem);
            }
            wait_vmem();
            __syncthreads();
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                qf[ks] = *reinterpret_cast<const u32x4*>(qlds + kq_off<D>(ra0 + l32, 2 * ks + hi));
            if (nxt >= 0) {
                // the next block's Q rows replace these once they are read
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                issue_q(nxt);
            }
        } else if constexpr (QN || QB) {
            // this wave's Q rows (past the sequence's length: zeros), read into
            // qf after the first tile's barrier
            int ln = lane;
            asm volatile("" : "+v"(ln));
#pragma unroll
            for (int k = 0; k < 32 / QRPC; ++k) {
                const int r = QRPC * k + ln / KCH, pc = ln % KCH;
                buf_to_lds16(Qb, qown + 1024 * k,
                             (uint32_t)(qw + r) * (D * 2) + (uint32_t)(kq_off<D>(ra0 + r, pc) - (ra0 + r) * D * 2));
            }
        } else {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) qf[ks] = Qb.load16((uint32_t)(q * D + 16 * ks + 8 * hi) * 2);
        }

        const int kv_len = q0 >= Nk ? 0 : (CAUSAL ? min(Nk, q0 + BR) : Nk);
        const int ntiles = (kv_len + BC - 1) / BC;
        const int nfull = min(min(CAUSAL ? q0 / BC : ntiles, Nk / BC), ntiles);

        auto issue_to = [&](unsigned char* base, int k0) {
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const int bi = wave + NW * i;
                const uint32_t rowb = (uint32_t)k0 * D * 2;
                buf_to_lds16(Kb, base + bi * 1024, rowb + cpk[i]);
                buf_to_lds16(Vb, base + TILE + bi * 1024, rowb + cpv[i]);
            }
        };
        // copies of tile jj into the buffer at base; past the last tile, the
        // next block's first tile (QL) or a tile past the end, which reads this
        // head's range or zeros and lands in the buffer no later tile reads
        auto issue_tile = [&](unsigned char* base, int jj) {
            if (!QL || jj < ntiles)
                issue_to(base, jj * BC);
            else if (nxt >= 0)
                issue_kv0(nxt, base);
        };
        // QN, QB: this wave's Q fragments from its rows of the Q tile (QB: then
        // a barrier, as the next copy goes to the buffer that holds them)
        auto read_qn = [&]() {
            if constexpr (QN || QB) {
#pragma unroll
                for (int ks = 0; ks < NKS; ++ks)
                    qf[ks] = *reinterpret_cast<const u32x4*>(qlds + kq_off<D>(ra0 + l32, 2 * ks + hi));
            }
            if constexpr (QB) __syncthreads();
        };

        const int g16 = lane >> 4;
        const int j16 = lane & 15;
        const int tr_row = 4 * hi + (j16 >> 2);
        const int tr_col = 2 * (16 * (g16 & 1) + 4 * (j16 & 3));

        // lane parts of the LDS addresses: K rows 32 kb + l32, chunk 2 ks + hi
        // (at d = 128 the swizzle depends on row & 15 only, so both halves share
        // them; at d = 64 it depends on row bit 5 too); V^T rows 16 kg + tr_row
        // (+ 8), bytes 64 db + tr_col
        constexpr int NKO = D == 128 ? 1 : 2;
        uint32_t ko[NKO][NKS], vo[NDB];
#pragma unroll
        for (int par = 0; par < NKO; ++par)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks)
                ko[par][ks] = lds_lane_off((uint32_t)kq_off<D>(32 * par + l32, 2 * ks + hi) - 32 * par * D * 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db) vo[db] = lds_lane_off((uint32_t)vt_off<D>(tr_row, 64 * db + tr_col));

        f32x16 o[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = zero16();
        float m_s = -INFINITY;
        float l_s = 0.f;

        // the 64 keys from k0 (sub-tile SUB of the tile in the buffer at cur)
        auto body = [&](int k0, auto mask_tag, auto sub_tag, const unsigned char* __restrict__ cur)
                        __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_tag)::value;
            constexpr int SUB = decltype(sub_tag)::value;
            const unsigned char* kbase = cur + SUB * 64 * D * 2;
            const unsigned char* vbase = cur + TILE + SUB * 64 * D * 2;

            auto kread = [&](int kb, int ks) {
                return *reinterpret_cast<const u32x4*>(kbase + ko[NKO == 1 ? 0 : (kb & 1)][ks] + 32 * kb * D * 2);
            };
            auto vread = [&](int kg, int db) {
                const u32x2 lo = lds_read_tr16(vbase + vo[db] + 16 * kg * D * 2);
                const u32x2 up = lds_read_tr16(vbase + vo[db] + (16 * kg + 8) * D * 2);
                return u32x4{lo[0], lo[1], up[0], up[1]};
            };
            // key k0 + 32 kb + acc_row(r, hi) is visible iff it is at most
            // min(q, N - 1) (without the causal mask: N - 1), i.e. iff the
            // register's constant part 8 (r / 4) + r % 4 is at most lim
            auto mask_half = [&](f32x16& s, int kb) {
                if (MASK) {
                    // (padded queries of a variable-length batch see no key)
                    const int lim = (SPARSE && q >= Nk) ? -1024
                                                         : (CAUSAL ? min(q, Nk - 1) : Nk - 1) - (k0 + 32 * kb) - 4 * hi;
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        if (8 * (r >> 2) + (r & 3) > lim) s[r] = -INFINITY;
                }
            };
            // probabilities of pair t (registers 2t, 2t + 1) of a half: dword
            // t & 3 of operand t >> 2 of that half
            auto exp_pair = [&](const f32x16& s, int t, float mu, float& ls, u32x4 (&pb)[2]) {
                const float p0 = fast_exp2(fmaf(s[2 * t], cl2, -mu));
                const float p1 = fast_exp2(fmaf(s[2 * t + 1], cl2, -mu));
                ls += p0 + p1;
                pb[t >> 2][t & 3] = Mma<T>::pack2(p0, p1);
            };
            // accept the half's probabilities, or move the maximum and redo them
            auto settle = [&](const f32x16& s, float& ls, u32x4 (&pb)[2]) {
                if (__any(!(m_s > -INFINITY && ls <= kSumCap))) {
                    float mx = -INFINITY;
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
                    const float mn = fmaxf(m_s, halves_max(mx) * cl2);
                    const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_s - mn);
                    l_s *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
#pragma unroll
                        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
                    m_s = mn;
                    const float mu = (m_s == -INFINITY) ? 0.f : m_s;
                    ls = 0.f;
#pragma unroll
                    for (int t = 0; t < 8; ++t) exp_pair(s, t, mu, ls, pb);
                }
                l_s += ls;
            };

            const float mu = (m_s == -INFINITY) ? 0.f : m_s;

            // Every LDS operand is read at least one step before its product
            // (each step below ends in a scheduling fence): K of the first half
            // up front, K of the second half under the first half's products, the
            // V^T operands of each half under the step before.
            u32x4 ka[NKS], kb2[NKS], va[2 * NDB], vb[2 * NDB];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) ka[ks] = kread(0, ks);

            // dropout: lane half hi draws the keep bytes of key block k0 / 32 + hi
            // of its row; the ten generator rounds run under the score products,
            // and one exchange between the halves gives every lane its bytes of
            // both blocks
            Philox4x64 pg;
            if constexpr (DROP) pg.start((uint32_t)(k0 / 32 + hi), (uint32_t)q, (uint32_t)(b * Hq + h), dp);

            // The wave's priority is raised while it issues the score products of
            // the first half and the second (whose slots carry the first half's
            // exponentials): when both waves of a SIMD are ready, the one feeding
            // the matrix cores issues first.
            __builtin_amdgcn_s_setprio(1);
            // scores of the first half | K reads of the second
            f32x16 s0 = zero16(), s1 = zero16();
            static_for<NKS>([&](auto tc) {
                constexpr int t = decltype(tc)::value;
                s0 = Mma<T>::mma(ka[t], qf[t], s0);
                kb2[t] = kread(1, t);
                if constexpr (DROP) pg.round();
                __builtin_amdgcn_sched_barrier(0);
            });
            mask_half(s0, 0);

            // scores of the second half | probabilities of the first | V^T reads
            // of the first half
            u32x4 pb0[2], pb1[2];
            float ls0 = 0.f, ls1 = 0.f;
            // With one probability pair per product (d = 128) the pairs run in a
            // three-stage pipeline over the steps: step t forms the exponent
            // arguments of pair t + 1, the exponentials of pair t and the sum and
            // packing of pair t - 1, so no step waits on its own chain.
            float ea[8][2], ee[8][2];
            auto arg = [&](const f32x16& sv, int t, float m) {
                ea[t][0] = fmaf(sv[2 * t], cl2, -m);
                ea[t][1] = fmaf(sv[2 * t + 1], cl2, -m);
            };
            auto ex = [&](int t) {
                ee[t][0] = fast_exp2(ea[t][0]);
                ee[t][1] = fast_exp2(ea[t][1]);
            };
            auto fin = [&](int t, float& ls, u32x4 (&pb)[2]) {
                ls += ee[t][0] + ee[t][1];
                pb[t >> 2][t & 3] = Mma<T>::pack2(ee[t][0], ee[t][1]);
            };
            if constexpr (PPB == 1) {
                arg(s0, 0, mu);
                static_for<NKS>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    s1 = Mma<T>::mma(kb2[t], qf[t], s1);
                    if constexpr (t + 1 < 8) arg(s0, t + 1, mu);
                    ex(t);
                    if constexpr (t > 0) fin(t - 1, ls0, pb0);
                    if (t < 2 * NDB) va[t] = vread(t / NDB, t % NDB);
                    if constexpr (DROP && NKS + t < 10) pg.round();
                    __builtin_amdgcn_sched_barrier(0);
                });
                fin(7, ls0, pb0);
            } else {
                static_for<NKS>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    s1 = Mma<T>::mma(kb2[t], qf[t], s1);
#pragma unroll
                    for (int u = 0; u < PPB; ++u) exp_pair(s0, PPB * t + u, mu, ls0, pb0);
                    if (t < 2 * NDB) va[t] = vread(t / NDB, t % NDB);
                    if constexpr (DROP && NKS + t < 10) pg.round();
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            __builtin_amdgcn_s_setprio(0);
            mask_half(s1, 1);
            settle(s0, ls0, pb0);
            // keep masks of both 32-key blocks: dword 2 t + jj / 2 holds the bytes
            // of pair (8 t + 2 jj, +1) of a block; the row sums above stay those
            // of the undropped probabilities
            uint32_t dm[2][4];
            auto drop_mask = [&](u32x4 (&pb)[2], const uint32_t (&m)[4]) {
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) pb[t][jj] &= drop_mask16x2(m[2 * t + (jj >> 1)], 2 * (jj & 1), dp.t8);
            };
            if constexpr (DROP) {
#pragma unroll
                for (int r = 2 * NKS; r < 10; ++r) pg.round();
                uint32_t w[8];
                pg.words(w);
                drop_pair_exchange(w, dm[0], dm[1]);
                drop_mask(pb0, dm[0]);
            }

            // P V of the first half | probabilities of the second | V^T reads of
            // the second half
            const float mu1 = (m_s == -INFINITY) ? 0.f : m_s;
            if constexpr (PPC == 1) {
                arg(s1, 0, mu1);
                static_for<2 * NDB>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    o[t % NDB] = Mma<T>::mma(va[t], pb0[t / NDB], o[t % NDB]);
                    if constexpr (t + 1 < 8) arg(s1, t + 1, mu1);
                    ex(t);
                    if constexpr (t > 0) fin(t - 1, ls1, pb1);
                    vb[t] = vread(2 + t / NDB, t % NDB);
                    __builtin_amdgcn_sched_barrier(0);
                });
                fin(7, ls1, pb1);
            } else {
                static_for<2 * NDB>([&](auto tc) {
                    constexpr int t = decltype(tc)::value;
                    o[t % NDB] = Mma<T>::mma(va[t], pb0[t / NDB], o[t % NDB]);
#pragma unroll
                    for (int u = 0; u < PPC; ++u) exp_pair(s1, PPC * t + u, mu1, ls1, pb1);
                    vb[t] = vread(2 + t / NDB, t % NDB);
                    __builtin_amdgcn_sched_barrier(0);
                });
            }
            settle(s1, ls1, pb1);
            if constexpr (DROP) drop_mask(pb1, dm[1]);

            // P V of the second half
#pragma unroll
            for (int t = 0; t < 2 * NDB; ++t) o[t % NDB] = Mma<T>::mma(vb[t], pb1[t / NDB], o[t % NDB]);
        };

        // tile j (its 64-key sub-tiles in turn; under the mask a wave skips the
        // sub-tiles above its rows)
        auto tile = [&](int j, auto mask_tag, const unsigned char* cur) __attribute__((always_inline)) {
            static_for<NSUB>([&](auto sc) {
                const int k0 = j * BC + 64 * decltype(sc)::value;
                if (!decltype(mask_tag)::value || !CAUSAL || k0 <= qw + 31) body(k0, mask_tag, sc, cur);
            });
        };

        bool compact = false;   // walk only the tiles a block mask allows
        if constexpr (SPARSE) compact = sp.mask != nullptr;
        if (compact) {
            const int nb = sp.nb;
            const unsigned char* mk = sp.mask + (size_t)(sp.heads == 1 ? 0 : h) * nb * nb;
            const int mr0 = min(q0 / 128, nb - 1);
            const int mr1 = min((q0 + BR - 1) / 128, nb - 1);
            // this wave's 32 rows lie in one mask row, and a 64-key tile in one
            // mask column: a wave computes a tile whole or not at all
            const unsigned char* mw = mk + min(qw / 128, nb - 1) * nb;
            // the next tile after jt that some row of the workgroup may see:
            // each lane of the wave tests one candidate, so a scan costs one
            // load latency per 64 tiles
            auto next = [&](int jt) {
                for (int base = jt + 1; base < ntiles; base += 64) {
                    const int c = base + lane;
                    bool any = false;
                    if (c < ntiles)
                        for (int r = mr0; r <= mr1; ++r) any |= mk[r * nb + c * BC / 128] != 0;
                    const uint64_t bal = __ballot(any);
                    if (bal) return base + __builtin_ctzll(bal);
                }
                return ntiles;
            };
            int jt = next(-1);
            if (jt < ntiles) issue_to(smem, jt * BC);
            wait_vmem();
            __syncthreads();
            read_qn();
            int par = 0;
            while (jt < ntiles) {
                const int jn = next(jt);
                // past the last allowed tile the copy reads this head's range or
                // zeros and lands in the buffer no later tile reads
                issue_to(smem + (par ^ 1) * STAGE, jn * BC);
                if (mw[jt * BC / 128] != 0 && (!CAUSAL || jt * BC <= qw + 31))
                    tile(jt, std::true_type{}, smem + par * STAGE);
                wait_vmem();
                __syncthreads();
                jt = jn;
                par ^= 1;
            }
        } else {
        if constexpr (!QL) {   // (QL: tile 0 is in buffer p0 already)
            issue_to(smem, 0);
            wait_vmem();
            __syncthreads();
            read_qn();
        }

        // The copy of the next tile is issued at the start of every tile, also the
        // last (issue_tile).  The pairs of unmasked tiles start in buffer 0; with
        // QL and p0 = 1, tile 0 (in buffer 1) runs alone first.
        int j = 0;
        if constexpr (QL) {
            if (p0 && nfull >= 1) {
                issue_tile(smem, 1);
                tile(0, std::false_type{}, smem + STAGE);
                wait_vmem();
                __syncthreads();
                j = 1;
            }
        }
        for (; j + 1 < nfull; j += 2) {
            issue_tile(smem + STAGE, j + 1);
            tile(j, std::false_type{}, smem);
            wait_vmem();
            __syncthreads();
            issue_tile(smem, j + 2);
            tile(j + 1, std::false_type{}, smem + STAGE);
            wait_vmem();
            __syncthreads();
        }
        for (; j < ntiles; ++j) {
            const int pj = (j + (QL ? p0 : 0)) & 1;
            issue_tile(smem + (pj ^ 1) * STAGE, j + 1);
            if (!CAUSAL || j * BC <= qw + 31) tile(j, std::true_type{}, smem + pj * STAGE);
            wait_vmem();
            __syncthreads();
        }
        }

        const float l_tot = l_s + swap_halves(l_s);
        if constexpr (QL) {
            // The wave's rows go through LDS: each lane writes its 8-byte pieces
            // in the swizzled layout of the Q tile, then reads back 16-byte
            // chunks in row order, so that each store writes 1 KB of consecutive
            // rows instead of 8 bytes in each of 32 rows.
            // (lane laundered as in issue_q: the staging addresses are formed
            // here, not held through the block loop)
            int ln = lane;
            asm volatile("" : "+v"(ln));
            // staging: the buffer of the block's last tile (free after the loops'
            // final barrier; the other holds the next block's first tile) for
            // waves 0 .. NW/2 - 1, the spare region for the others
            unsigned char* const ost = wave < NW / 2
                                           ? smem + ((ntiles - 1 + p0) & 1) * STAGE + wave * OWAVE
                                           : smem + 2 * STAGE + QTILE + (wave - NW / 2) * OWAVE;
            const float inv = 1.f / l_tot;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = Mma<T>::pack2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
                    w[1] = Mma<T>::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(ost + kq_off<D>(ln & 31, 4 * db + g) + 8 * (ln >> 5)) = w;
                }
            uint16_t* Ow = O + qoff + (size_t)qw * D;
#pragma unroll
            for (int k = 0; k < 32 / QRPC; ++k) {
                const int r = QRPC * k + ln / KCH;
                const u32x4 v = *reinterpret_cast<const u32x4*>(ost + kq_off<D>(r, ln % KCH));
                if (qw + r < N) *reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(Ow) + 1024 * k + 16 * ln) = v;
            }
            if (q < N && hi == 0) LSE[(size_t)(b * Hq + h) * N + q] = (m_s + __log2f(l_tot)) * kLn2;
            p0 = (ntiles + p0) & 1;   // where the next block's tile 0 went
        } else if constexpr (QN || QB) {
            // as above, staged in the wave's own Q rows; rows that see no key
            // (padding) get O = 0 and lse = -inf, kept probabilities are scaled
            // by 256 / t8
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const bool empty = SPARSE && (!(l_tot > 0.f) || q >= Nk);
            const float inv = empty ? 0.f : (DROP ? dp.scale : 1.f) / l_tot;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = Mma<T>::pack2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
                    w[1] = Mma<T>::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(qlds + kq_off<D>(ra0 + (ln & 31), 4 * db + g) + 8 * (ln >> 5)) = w;
                }
            unsigned char* const Ow = reinterpret_cast<unsigned char*>(O + qoff + (size_t)qw * D);
#pragma unroll
            for (int k = 0; k < 32 / QRPC; ++k) {
                const int r = QRPC * k + ln / KCH;
                const u32x4 v = *reinterpret_cast<const u32x4*>(qlds + kq_off<D>(ra0 + r, ln % KCH));
                if (qw + r < N) *reinterpret_cast<u32x4*>(Ow + 1024 * k + 16 * ln) = v;
            }
            if (q < N && hi == 0) LSE[(size_t)(b * Hq + h) * N + q] = empty ? -INFINITY : (m_s + __log2f(l_tot)) * kLn2;
        } else if (q < N) {
            // rows that see no key (block masks, padding) get O = 0 and lse = -inf;
            // kept probabilities are scaled by 256 / t8 here
            const bool empty = SPARSE && (!(l_tot > 0.f) || q >= Nk);
            const float inv = empty ? 0.f : (DROP ? dp.scale : 1.f) / l_tot;
            uint16_t* Orow = O + qoff + (size_t)q * D;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 w;
                    w[0] = Mma<T>::pack2(o[db][4 * g] * inv, o[db][4 * g + 1] * inv);
                    w[1] = Mma<T>::pack2(o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv);
                    *reinterpret_cast<u32x2*>(Orow + 32 * db + 8 * g + 4 * hi) = w;
                }
            if (hi == 0) LSE[(size_t)(b * Hq + h) * N + q] = empty ? -INFINITY : (m_s + __log2f(l_tot)) * kLn2;
        }
    }
    FA355_CLOCK_END(fa355_clock_fwd)
}

// fp32 inputs: the same walk with the fp32 matrix-core op (32x32x2), P kept in
// fp32, single-buffered tiles of 32 keys.  Four waves, 128 rows per workgroup.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
fwd32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
             float* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int N, float cl2) {
    constexpr int NW = 4;
    constexpr int BR = 32 * NW;
    constexpr int BC = 32;
    constexpr int KS = D + 1;  // padded K row (column reads)
    constexpr int NDB = D / 32;
    __shared__ float Ks[BC * KS];
    __shared__ float Vs[BC * D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // provably wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int nqb = (N + BR - 1) / BR;
    const int total = nqb * Hq * B;
    const int logical = xcd_remap((int)blockIdx.x, total);
    const int qb_raw = logical % nqb;
    const int bh = logical / nqb;
    const int qb = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int hk = h / (Hq / Hkv);
    const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
    const size_t koff = ((size_t)b * Hkv + hk) * (size_t)N * D;

    const int q0 = qb * BR;
    const int qw = q0 + 32 * wave;
    const int q = qw + l32;

    float qf[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = (q < N) ? Q[qoff + (size_t)q * D + 2 * ks + hi] : 0.f;

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero16();
    float m_s = -INFINITY, l_s = 0.f;

    const int kv_len = CAUSAL ? min(N, q0 + BR) : N;
    for (int k0 = 0; k0 < kv_len; k0 += BC) {
        __syncthreads();
        for (int i = tid; i < BC * D; i += 256) {
            const int r = i / D, c = i % D;
            const int key = k0 + r;
            const float kv = key < N ? K[koff + (size_t)key * D + c] : 0.f;
            const float vv = key < N ? V[koff + (size_t)key * D + c] : 0.f;
            Ks[r * KS + c] = kv;
            Vs[r * D + c] = vv;
        }
        __syncthreads();
        if (CAUSAL && k0 > qw + 31) continue;

        f32x16 s = zero16();
#pragma unroll 8
        for (int ks = 0; ks < D / 2; ++ks) s = mma_f32(Ks[l32 * KS + 2 * ks + hi], qf[ks], s);

#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = k0 + acc_row(r, hi);
            if ((CAUSAL && key > q) || key >= N) s[r] = -INFINITY;
        }
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
        mx = fmaxf(mx, swap_halves(mx));
        const float mt = mx * cl2;
        if (__any(mt > m_s + kTau)) {
            const float mn = fmaxf(m_s, mt);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_s - mn);
            l_s *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
            m_s = mn;
        }
        const float mu = (m_s == -INFINITY) ? 0.f : m_s;
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            p[r] = fast_exp2(fmaf(s[r], cl2, -mu));
            l_s += p[r];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                o[db] = mma_f32(Vs[acc_row(r, hi) * D + 32 * db + l32], p[r], o[db]);
    }

    const float l_tot = l_s + swap_halves(l_s);
    if (q < N) {
        const float inv = 1.f / l_tot;
        float* Orow = O + qoff + (size_t)q * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
                for (int i = 0; i < 4; ++i) w[i] = o[db][4 * g + i] * inv;
                *reinterpret_cast<f32x4*>(Orow + 32 * db + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) LSE[(size_t)(b * Hq + h) * N + q] = (m_s + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D, bool CAUSAL, int NW, int BC, bool PERSIST = false, bool DROP = false,
          bool SPARSE = false, int GS = 1>
hipError_t launch16v6(const FwdArgs& a) {
    constexpr int BR = 32 * NW / GS;
    const int nqb = (a.N + BR - 1) / BR;
    const long long total = (long long)nqb * (a.Hq / GS) * a.B;
    int grid = 0;
    if constexpr (PERSIST) {
        // workgroups resident per compute unit for this instantiation
        static const int per_cu = [] {
            int n = 0;
            return hipOccupancyMaxActiveBlocksPerMultiprocessor(
                       &n, reinterpret_cast<const void*>(fwd16v6_kernel<T, D, CAUSAL, NW, BC, true, DROP, SPARSE, GS>),
                       NW * 64, 0) == hipSuccess ? n : 0;
        }();
        grid = persistent_grid() * per_cu;
    }
    if constexpr (PERSIST) {
        if (grid >= 8 && total > grid) {
            hipLaunchKernelGGL((fwd16v6_kernel<T, D, CAUSAL, NW, BC, true, DROP, SPARSE, GS>), dim3((unsigned)grid),
                               dim3(NW * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                               (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, a.cl2, a.dp,
                               a.sp, fwd_pool_slot());
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((fwd16v6_kernel<T, D, CAUSAL, NW, BC, false, DROP, SPARSE, GS>), dim3((unsigned)total),
                       dim3(NW * 64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k,
                       (const uint16_t*)a.v, (uint16_t*)a.o, a.lse, a.B, a.Hq, a.Hkv, a.N, a.cl2, a.dp, a.sp,
                       nullptr);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch32(const FwdArgs& a) {
    const int nqb = (a.N + 127) / 128;
    const long long total = (long long)nqb * a.Hq * a.B;
    hipLaunchKernelGGL((fwd32_kernel<D, CAUSAL>), dim3((unsigned)total), dim3(256), 0, a.stream,
                       (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse,
                       a.B, a.Hq, a.Hkv, a.N, a.cl2);
    return hipGetLastError();
}

// Kernel choice: the sixth generation throughout.  d = 128: eight 32-row waves
// (one workgroup per compute unit, two waves per SIMD; the pipelined halves
// give each wave its own overlap of matrix and vector work, and eight waves
// halve the copies per wave and the L2 traffic per query row), on the
// persistent grid.  d = 64: four waves and 64-key tiles (three waves per SIMD
// fit in the registers), on the persistent grid under the causal mask only
// (without it, one row block per workgroup measures faster at this head
// dimension).  Dropout, block masks and variable lengths are compile-time
// variants of the same kernels.
template <typename T, int D, bool CAUSAL>
hipError_t dispatch16c(const FwdArgs& a) {
    constexpr int NW = D == 128 ? FA355_FWD_NW128 : 4;
    constexpr bool PERS = FA355_FWD_PERSIST && (D == 128 || CAUSAL);
    // (with dropout the persistent round loop pushes the d = 128 build past the
    // register file, so each row block gets a workgroup of its own)
    if (a.drop) return launch16v6<T, D, CAUSAL, NW, 64, D == 64 && CAUSAL, true>(a);
    // block masks: 128-row blocks (four waves), one mask row per workgroup, so
    // that no wave waits through the tiles that only another mask row allows;
    // sequence lengths alone keep the dense tiling.  Both take one workgroup
    // per row block: their work per row block varies with the mask and the
    // lengths, which the hardware's dispatch balances and a static schedule
    // does not.
    if (a.sparse && a.sp.mask) return launch16v6<T, D, CAUSAL, 4, 64, false, false, true>(a);
    if (a.sparse) return launch16v6<T, D, CAUSAL, NW, 64, false, false, true>(a);
#if FA355_FWD_STACK
    // grouped K/V heads at d = 128: one workgroup takes the same rows of 2 or 4
    // query heads of a group, which then share every K/V tile it stages
    // (a stacking factor is used only where each head's row block, 32 NW / GS
    // rows, stays a multiple of the key tile)
    if constexpr (D == 128) {
        constexpr int BCD = FA355_FWD_BC128;
        const int G = a.Hq / a.Hkv;
        if constexpr ((32 * NW / 4) % BCD == 0)
            if (G % 4 == 0) return launch16v6<T, D, CAUSAL, NW, BCD, PERS, false, false, 4>(a);
        if constexpr ((32 * NW / 2) % BCD == 0)
            if (G % 2 == 0) return launch16v6<T, D, CAUSAL, NW, BCD, PERS, false, false, 2>(a);
    }
#endif
    return launch16v6<T, D, CAUSAL, NW, (D == 128 ? FA355_FWD_BC128 : 64), PERS>(a);
}

template <typename T, int D>
hipError_t dispatch16(const FwdArgs& a) {
    return a.causal ? dispatch16c<T, D, true>(a) : dispatch16c<T, D, false>(a);
}

template <int D>
hipError_t dispatch32(const FwdArgs& a) {
    return a.causal ? launch32<D, true>(a) : launch32<D, false>(a);
}

}  // namespace

hipError_t launch_fwd(const FwdArgs& a) {
    switch (a.dtype) {
        case 2: return a.d == 64 ? dispatch16<BF16, 64>(a) : dispatch16<BF16, 128>(a);
        case 1: return a.d == 64 ? dispatch16<FP16, 64>(a) : dispatch16<FP16, 128>(a);
        default: return a.d == 64 ? dispatch32<64>(a) : dispatch32<128>(a);
    }
}

}  // namespace fa355
