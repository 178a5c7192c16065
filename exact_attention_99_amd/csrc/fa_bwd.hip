// Backward pass of exact tiled attention with recomputation, gfx950.
//
// Gradients of sum(dO * O) for O = softmax(scale * Q K^T [causal]) V.  The
// pages state only that the backward pass rebuilds the attention matrix from
// Q, K, V and the saved softmax statistics instead of storing it
// ("FlashAttention Kernel" glossary, Recomputation bullet; "FlashAttention"
// glossary, recomputation paragraph); the gradient formulas are the chain
// rule through O = P V and the row-wise softmax:
//
//   D_i = sum_k dO_ik O_ik          P = exp(scale * Q K^T - lse)
//   dP  = dO V^T                    dS = P * (dP - D)
//   dV  = P^T dO     dK = scale * dS^T Q     dQ = scale * dS K
//
// Three launches on the caller's stream:
//   1. delta:  D_i for every query row (memory bound, one pass over O, dO).
//   2. dkdv:   one workgroup per block of 128 keys of one K/V head; each wave
//              owns 32 keys and keeps their dK^T, dV^T in fp32 registers while
//              it walks all query blocks of every query head of the group
//              (the key-block-outer order of the "FlashAttention Kernel"
//              glossary's Tiling bullet).  Scores are formed as S = Q K^T so
//              that a lane owns one key: P and dS are then directly the B
//              operands of dV^T += dO^T P and dK^T += Q^T dS.
//   3. dq:     one workgroup per block of query rows (query-outer, like the
//              forward pass); S^T = K Q^T and dP^T = V dO^T give a lane one
//              query, and dS^T is directly the B operand of dQ^T += K^T dS^T.
// P and dP are thus formed twice (once per pass), which replaces fp32 atomic
// accumulation of dQ across key blocks; every result is written exactly once.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa355 {

FA355_CLOCK_PROBE_ARRAY(fa355_clock_bwd)

// Counters of the persistent dK/dV pass's shared tail: a ring of 64-byte slots
// (a claim counter per XCD and a done counter each), one slot per launch,
// chosen round-robin on the host; a launch leaves its slot at zero when it ends, so
// launches on other streams stay apart while fewer than kPoolSlots of them
// are in flight on one device at once.
constexpr int kPoolSlots = 64;
__device__ __attribute__((aligned(64))) unsigned fa355_dkdv_pool[kPoolSlots * 16];

// This launch's slot on the current device (nullptr if the symbol's address
// cannot be had: the kernel then keeps its static schedule).
unsigned* dkdv_pool_slot() {
    static std::atomic<unsigned*> base[64];
    static std::atomic<unsigned> seq{0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    unsigned* p = base[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(fa355_dkdv_pool)) != hipSuccess || !a) return nullptr;
        p = static_cast<unsigned*>(a);
        base[dev].store(p, std::memory_order_release);
    }
    return p + 16 * (seq.fetch_add(1, std::memory_order_relaxed) % kPoolSlots);
}

namespace {

// ---------------------------------------------------------------------------
// D_i = sum_k dO_ik O_ik, fp32 accumulation.  D/8 (16-bit) or D/4 (fp32)
// lanes share a row and reduce with cross-lane adds.
template <typename T, int D>
__global__ void __launch_bounds__(256)
delta16_kernel(const uint16_t* __restrict__ O, const uint16_t* __restrict__ dO,
               float* __restrict__ Delta, long long rows) {
    constexpr int LPR = D / 8;
    constexpr int RPB = 256 / LPR;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const u32x4 a = ld_global16(O + row * D + 8 * c);
        const u32x4 g = ld_global16(dO + row * D + 8 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc = fmaf(Mma<T>::to_f32(a[i] & 0xffffu), Mma<T>::to_f32(g[i] & 0xffffu), acc);
            acc = fmaf(Mma<T>::to_f32(a[i] >> 16), Mma<T>::to_f32(g[i] >> 16), acc);
        }
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) Delta[row] = acc;
}

template <int D>
__global__ void __launch_bounds__(256)
delta32_kernel(const float* __restrict__ O, const float* __restrict__ dO, float* __restrict__ Delta,
               long long rows) {
    constexpr int LPR = D / 4;
    constexpr int RPB = 256 / LPR;
    const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
    const int c = threadIdx.x % LPR;
    float acc = 0.f;
    if (row < rows) {
        const f32x4 a = *reinterpret_cast<const f32x4*>(O + row * D + 4 * c);
        const f32x4 g = *reinterpret_cast<const f32x4*>(dO + row * D + 4 * c);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(a[i], g[i], acc);
    }
#pragma unroll
    for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (row < rows && c == 0) Delta[row] = acc;
}

// ---------------------------------------------------------------------------
// Segment seg of a dK/dV query tile of NQB blocks: 0 and the odd segments
// before the last hold the S/dP products of block (seg + 1) / 2; the others the
// dV/dK products of block seg / 2 - 1, and the last one those of block NQB - 1.
template <int NQB>
__host__ __device__ constexpr bool dkdv_seg_is_s(int seg) {
    return seg == 0 || ((seg & 1) && seg < 2 * NQB - 1);
}
template <int NQB>
__host__ __device__ constexpr int dkdv_seg_block(int seg) {
    return dkdv_seg_is_s<NQB>(seg) ? (seg + 1) / 2 : (seg == 2 * NQB - 1 ? NQB - 1 : seg / 2 - 1);
}

// ---------------------------------------------------------------------------
// Software-pipelined dK / dV kernel.  Four waves, 128 keys per workgroup (32
// per wave, one per lane), query rows in steps.  The Q and dO tiles arrive in
// LDS through buffer-to-LDS copies (no staging registers) and are stored
// row-major only, with a swizzle that suits both ways they are read: 128-bit
// reads of 16 consecutive rows for the A operands of S = Q K^T and
// dP = dO V^T, and transposing reads for the A operands of dV^T += dO^T P and
// dK^T += Q^T dS.  One wave per SIMD (the dK/dV
// accumulators and the K/V operands fill most of the register file), so the
// overlap of matrix work, softmax arithmetic and LDS traffic has to come from
// the instruction order of a single wave.  A query tile of NQB 32-row blocks
// is one fixed sequence of MFMA slots:
//   S/dP(0) | S/dP(1) | dV,dK(0) | S/dP(2) | dV,dK(1) | ... | dV,dK(NQB-1)
// Every slot's A operand (a Q or dO row chunk for S/dP, a pair of transposing
// dO^T or Q^T reads for dV/dK) is read from LDS a fixed number of slots ahead,
// so only a small window of operands is live.  The softmax and dS arithmetic
// of block b runs in the slots of the dV/dK products of block b-1 (block 0's
// runs between the first two segments), and block b's row terms are read
// during its S/dP segment.  Query tiles (Q, dO) of 16384/D rows are
// double-buffered in LDS and filled by buffer-to-LDS copies.  Rows past N read
// as zeros (Q, dO, the logsumexp and D row terms alike), which makes their
// P * (dP - D) and P^T dO contributions exactly zero, and keys past N are never
// written back, so only the causal condition needs a mask.
//
// MASKED = 1: variable lengths.  Everything past the sequence's length reads as
// zeros like the rows past N above, and the dK and dV of keys past it are
// written as zeros.  MASKED = 2: block masks (and lengths).  The workgroup's 128
// keys are one mask column: the walk visits only the steps whose query rows
// meet a set mask block, all through the masked path, with one allow bit per
// 32-row block.
//
// DROP: attention dropout (fa_common.h): dV^T += dO^T (Z P 256 / t8) and
// dS = P * (Z dP 256 / t8 - D).  A wave's 32 keys are one key block, so each
// query row of a step needs one generator call: lane l draws rows q0 + l and
// q0 + 64 + l.  The ten rounds of the next step's calls run in the slots of
// the step's last segment, the one without softmax work (spreading them over
// the S/dP segments as well made the compiler fail); at the end of the step
// the bytes go to the wave's LDS area, and transposing byte reads, issued in
// each block's S/dP segment, give every lane the bytes of its key for its 16
// rows.  At d = 64 the query tile has 128 rows under dropout, so that the byte
// areas fit in LDS beside the double-buffered tiles.
template <typename T, int D, bool CAUSAL, bool PERSIST = false, int MASKED = 0, bool DROP = false>
__global__ void __launch_bounds__(256)
dkdv16v3_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
                const float* __restrict__ LSE, const float* __restrict__ Delta,
                uint16_t* __restrict__ dK, uint16_t* __restrict__ dV, int B, int Hq, int Hkv, int N,
                float cl2, float scale, DropParams dp, SparseParams sp, unsigned* __restrict__ pool) {
    FA355_CLOCK_BEGIN
    static_assert(!(DROP && MASKED), "dropout runs on the dense walk");
    constexpr int NW = 4;
    constexpr int BKV = 128;
    constexpr int BQ = (DROP && D == 64) ? 128 : (D == 128 ? FA355_DKDV_BQ128 : 256);
    constexpr int NQB = BQ / 32;
    constexpr int KCH = D / 8;
    constexpr int TB = BQ * D * 2;
    constexpr int OFF_DOS = TB;
    constexpr int OFF_LSE = 2 * TB;
    constexpr int OFF_DL = OFF_LSE + BQ * 4;
    constexpr int STAGE = OFF_DL + BQ * 4;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr int WI = TB / 1024;
    static_assert(WI % NW == 0, "tile copies split evenly over the waves");
    constexpr int IPW = WI / NW;
    static_assert(BQ <= 256, "row terms staged one per thread");
    static_assert(BQ >= BKV, "only a key block's first query tile meets its diagonal");
    constexpr bool SPARSE = MASKED != 0;
    constexpr bool BLOCKMASK = MASKED == 2;
    constexpr int NSLOT = 2 * NKS;          // MFMAs per segment (== 4 * NDB)
    static_assert(NSLOT == 4 * NDB, "S/dP and dV/dK segments hold the same MFMA count");
    constexpr int EPS = 16 / NSLOT;         // softmax elements per slot
    constexpr int NSEG = 2 * NQB;
    constexpr int TSLOT = NSEG * NSLOT;
    constexpr int AHEAD = FA355_DKDV_AHEAD;  // operand read distance, in slots
    // dropout: generator calls per lane and step, and their rounds
    constexpr int NCALL = BQ / 64;
    constexpr int NROUND = 10 * NCALL;
    constexpr int DROP_AREA = BQ * 32;      // per wave: BQ rows x 32 keys

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE + (DROP ? NW * DROP_AREA : 0)];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int nkb = (N + BKV - 1) / BKV;
    const int total = nkb * Hkv * B;
    // Shared tail (dense causal walk, with a pool slot), as in the forward: the
    // first rs rounds are static, the key blocks past them in each XCD's range
    // are claimed one at a time (claim_pooled: own XCD's pool first, the
    // longest first: key block 0 of a head meets every query row), so XCDs at
    // lower clocks take fewer.
    // The claimed index passes through the row-term area of buffer kvbuf
    // (below), which no copy of the block reaches before its K and V rows are
    // read, after every wave has read the index.
    constexpr bool TAIL = PERSIST && CAUSAL && !DROP && !SPARSE;
    const int gxd = (int)gridDim.x / 8;
    const int rounds_x = gxd > 0 ? (total / 8) / gxd : 0;
    const int tail_rounds = max(2, rounds_x / 8);
    // (the 16-bit pool counters: each pool holds at most (tail_rounds + 1) G/8
    // blocks, its back counter counts at most all pooled claims and one failed
    // claim per workgroup)
    const bool fits16 = 9 * (tail_rounds + 1) * gxd + (int)gridDim.x < (1 << 16);
    const int rs = (TAIL && pool && fits16) ? max(0, rounds_x - tail_rounds) : 0x7fffffff;
    // One key block per workgroup, or (PERSIST) a grid of one workgroup per
    // compute unit that walks its key blocks in rounds.
    for (int round = 0;; ++round) {
        int logical;
        if constexpr (PERSIST) {
            if (round < rs) {
                logical = persist_block((int)blockIdx.x, (int)gridDim.x, total, round);
                if (logical < 0) break;
            } else {
                if constexpr (TAIL) {
                    int* const word = reinterpret_cast<int*>(smem + (((Hq / Hkv) & 1) ^ 1) * STAGE + OFF_LSE);
                    __syncthreads();
                    if (tid == 0)
                        *word = claim_pooled(pool, (int)blockIdx.x % 8, total, rs * gxd, nkb, gridDim.x);
                    __syncthreads();
                    logical = __builtin_amdgcn_readfirstlane(*reinterpret_cast<volatile int*>(word));
                    if (logical < 0) break;
                } else {
                    break;
                }
            }
        } else {
            if (round > 0) break;
            logical = xcd_remap((int)blockIdx.x, total);
        }
        const int jb = logical % nkb;
        const int bhk = logical / nkb;
        // the masked path takes the batch index fastest (XCD balance across
        // sequences of different lengths)
        const int hk = SPARSE ? bhk / B : bhk % Hkv;
        const int b = SPARSE ? bhk % B : bhk / Hkv;
        const int G = Hq / Hkv;

        const int kv0 = jb * BKV;
        const int kw = kv0 + 32 * wave;
        const int key = kw + l32;
        const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)N * D;
        // valid positions of this sequence (the masked path's lengths; else N)
        const int Nk = (SPARSE && sp.seqlens) ? min(max(sp.seqlens[b], 0), N) : N;
        const uint32_t head_bytes = (uint32_t)Nk * D * 2;

        // This wave's 32 K and V rows arrive by coalesced buffer-to-LDS copies
        // (1 KB of consecutive rows each, stored with the K tiles' swizzle)
        // into its own 16 KB of the buffer the first step does not use, and are
        // read from there into registers between two barriers (the second keeps
        // the next step's copies from overwriting another wave's rows early).
        // (Loaded directly, a lane's 16-byte pieces lie 256 bytes apart: every
        // load touches 32 cache lines.)  Keys past the sequence read zeros.
        constexpr int KRPC = 1024 / (D * 2);   // rows per 1 KB copy
        const int kvbuf = BLOCKMASK ? 1 : ((CAUSAL && kv0 < Nk ? Hq / Hkv : 0) & 1) ^ 1;
        unsigned char* const kvst = smem + kvbuf * STAGE + wave * (2 * 32 * D * 2);
        {
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const Buf Kb(K + kvoff, head_bytes), Vb(V + kvoff, head_bytes);
#pragma unroll
            for (int k = 0; k < 32 / KRPC; ++k) {
                const int r = KRPC * k + ln / KCH, pc = ln % KCH;
                const uint32_t src = (uint32_t)kw * D * 2 + (uint32_t)kq_off<D>(r, pc);
                buf_to_lds16(Kb, kvst + 1024 * k, src);
                buf_to_lds16(Vb, kvst + 32 * D * 2 + 1024 * k, src);
            }
        }
        u32x4 kf[NKS], vf[NKS];
        auto read_kv = [&]() {
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                kf[ks] = *reinterpret_cast<const u32x4*>(kvst + kq_off<D>(l32, 2 * ks + hi));
                vf[ks] = *reinterpret_cast<const u32x4*>(kvst + 32 * D * 2 + kq_off<D>(l32, 2 * ks + hi));
            }
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                // keep the B operands in the accumulation registers, leaving the
                // vector registers to the pipeline
                asm volatile("" : "+a"(kf[ks]));
                asm volatile("" : "+a"(vf[ks]));
            }
        };

        f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            dkt[db] = zero16();
            dvt[db] = zero16();
        }

        const int qb_first = CAUSAL ? kv0 / BQ : 0;
        const int qb_count = kv0 >= Nk ? 0 : (Nk + BQ - 1) / BQ - qb_first;
        const int nsteps = G * qb_count;

        uint32_t cp[IPW];
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int p = (wave + NW * i) * 64 + lane;
            const int row = p / KCH, pc = p % KCH;
            cp[i] = (uint32_t)(row * D * 2 + 16 * (pc ^ dual_swz<D>(row)));
        }
        float sl = 0.f, sd = 0.f;

        // Tile order: under a causal mask the G diagonal tiles (the first query
        // tile of each head, the only ones that need the mask) come first, then
        // the remaining tiles head by head.
        const int ndiag = (CAUSAL && qb_count > 0) ? G : 0;
        const int nrest = qb_count - (CAUSAL ? 1 : 0);
        auto step_rows = [&](int s, int& h, int& q0) {
            if (CAUSAL && s < ndiag) {
                h = hk * G + s;
                q0 = qb_first * BQ;
            } else {
                const int m = s - ndiag;
                h = hk * G + m / nrest;
                q0 = (qb_first + (CAUSAL ? 1 : 0) + m % nrest) * BQ;
            }
        };
        // LDS buffer of tile s: the last diagonal tile uses buffer 1, so that the
        // remaining tiles alternate 0, 1, 0, ... from their first one
        auto buf_of = [&](int s) { return (s < ndiag ? ndiag - s : s - ndiag) & 1; };
        auto issue = [&](int s, int buf) {
            int h, q0;
            step_rows(s, h, q0);
            const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
            const Buf Qb(Q + qoff, head_bytes), Db(dO + qoff, head_bytes);
            unsigned char* base = smem + buf * STAGE;
#pragma unroll
            for (int i = 0; i < IPW; ++i) {
                const uint32_t off = (uint32_t)q0 * D * 2 + cp[i];
                buf_to_lds16(Qb, base + (wave + NW * i) * 1024, off);
                buf_to_lds16(Db, base + OFF_DOS + (wave + NW * i) * 1024, off);
            }
            const size_t roff = ((size_t)b * Hq + h) * (size_t)N;
            if (tid < BQ) {
                // scaled to base 2 when it is published (a use here would make the
                // wave wait for the tile copies issued just before)
                sl = Buf(LSE + roff, (uint32_t)Nk * 4).load_f32((uint32_t)(q0 + tid) * 4);
                sd = Buf(Delta + roff, (uint32_t)Nk * 4).load_f32((uint32_t)(q0 + tid) * 4);
            }
        };
        auto put_rows = [&](int buf) {
            unsigned char* base = smem + buf * STAGE;
            if (tid < BQ) {
                reinterpret_cast<float*>(base + OFF_LSE)[tid] = sl * kLog2e;
                reinterpret_cast<float*>(base + OFF_DL)[tid] = sd;
            }
        };

        const int g16 = lane >> 4;
        const int j16 = lane & 15;
        const int tr_row = 4 * hi + (j16 >> 2);
        const int tr_col = 2 * (16 * (g16 & 1) + 4 * (j16 & 3));

        // dropout: the generator calls of one step (rows q0 + 64 c + lane of
        // head h, this wave's key block) and the wave's byte area
        Philox4x64 pg[DROP ? NCALL : 1];
        unsigned char* const dbase = smem + 2 * STAGE + (DROP ? wave * DROP_AREA : 0);
        auto drop_start = [&](int st) {
            if constexpr (DROP) {
                int h, q0;
                step_rows(st, h, q0);
#pragma unroll
                for (int c = 0; c < NCALL; ++c)
                    pg[c].start((uint32_t)(kw / 32), (uint32_t)(q0 + 64 * c + lane), (uint32_t)(b * Hq + h), dp);
            }
        };
        auto drop_store = [&](unsigned char* dr) {
            if constexpr (DROP) {
#pragma unroll
                for (int c = 0; c < NCALL; ++c) {
                    uint32_t w[8];
                    pg[c].words(w);
                    *reinterpret_cast<u32x4*>(dr + (64 * c + lane) * 32) = u32x4{w[0], w[1], w[2], w[3]};
                    *reinterpret_cast<u32x4*>(dr + (64 * c + lane) * 32 + 16) = u32x4{w[4], w[5], w[6], w[7]};
                }
            }
        };

        // Segment seg of a tile: 0 and odd segments before the last hold the S/dP
        // products of block (seg + 1) / 2; the others the dV/dK products of block
        // seg / 2 - 1, and the last one those of block NQB - 1.
        // mlim: element (block blk, row offset o) of this lane is visible when
        // 32 blk + o >= mlim (causal: the query row is at or after the key) and
        // (block masks) bit blk of allow is set
        // rt_base: the tile's buffer.  Every LDS read of the step goes through
        // this restrict-qualified pointer, so the transposing reads carry alias
        // information and the compiler does not make them wait for the copies of
        // the next step into the other buffer.
        // (The buffer is a run-time argument of the step, not a template one: a
        // step specialised on a constant buffer would lose that information.)
        // sn: the step whose dropout bytes this step draws, dr: the wave's byte
        // area (DROP; restrict-qualified like the buffer, for the same reason)
        auto run_step = [&](auto mask_tag, const unsigned char* __restrict__ rt_base, int mlim,
                            uint32_t allow, int sn, unsigned char* __restrict__ dr) __attribute__((always_inline)) {
            constexpr bool MASK = decltype(mask_tag)::value;
            // The lane-dependent parts of every LDS address, with the buffer's base
            // folded in, are formed once per tile; each read then adds only an
            // immediate (block, half and tensor offsets), which stays within the
            // 16-bit offset field of the LDS instructions (the buffer base is a
            // constant once the step is inlined into the unmasked loop).
            const uint32_t bb = (uint32_t)(rt_base - smem);
            uint32_t ao[NKS], to[2][NDB];
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) ao[ks] = lds_lane_off(bb + dual_off<D>(l32, 16 * (2 * ks + hi)));
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    to[u][db] = lds_lane_off(bb + dual_off<D>(8 * u + tr_row, 64 * db + tr_col));
            const uint32_t ro = lds_lane_off(bb + OFF_LSE + 16 * hi);

            u32x4 op[TSLOT];
            f32x16 sacc = zero16(), dpacc = zero16();
            u32x4 pb[2][2], dsb[2][2];
            f32x4 lc[4], dc[4];
            uint32_t md[4];   // DROP: keep bytes of the current block, dword g
            drop_start(sn);

            auto load_op = [&](auto nc) {
                constexpr int n = decltype(nc)::value;
                constexpr int seg = n / NSLOT, j = n % NSLOT;
                constexpr int blk = dkdv_seg_block<NQB>(seg);
                if constexpr (dkdv_seg_is_s<NQB>(seg)) {
                    constexpr int ks = j >> 1;
                    constexpr int imm = ((j & 1) ? OFF_DOS : 0) + 32 * blk * D * 2;
                    op[n] = *reinterpret_cast<const u32x4*>(rt_base + (ao[ks] - bb) + imm);
                } else {
                    constexpr int t = j / (2 * NDB), db = (j >> 1) % NDB;
                    constexpr int imm = ((j & 1) ? 0 : OFF_DOS) + (32 * blk + 16 * t) * D * 2;
                    const u32x2 lo = lds_read_tr16(rt_base + (to[0][db] - bb) + imm);
                    const u32x2 up = lds_read_tr16(rt_base + (to[1][db] - bb) + imm);
                    op[n] = u32x4{lo[0], lo[1], up[0], up[1]};
                }
            };
            auto load_rows = [&](int blk, int k) {
                const int g = k >> 1;
                const int imm = 4 * (32 * blk + 8 * g);
                if (k & 1)
                    dc[g] = *reinterpret_cast<const f32x4*>(rt_base + (ro - bb) + (OFF_DL - OFF_LSE) + imm);
                else
                    lc[g] = *reinterpret_cast<const f32x4*>(rt_base + (ro - bb) + imm);
            };
            // keep bytes of rows 8 g .. 8 g + 7 of block blk at this lane's key:
            // register 4 g + i (row 8 g + 4 hi + i) is byte i of dword hi
            auto load_drop = [&](int blk, int g) {
                const int s16 = lane & 15;
                const int off = (32 * blk + 8 * g + (s16 >> 1)) * 32 + 16 * ((lane >> 4) & 1) + 8 * (s16 & 1);
                const i32x2 x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                    (__attribute__((address_space(3))) i32x2*)(dr + off));
                md[g] = (uint32_t)(hi ? x[1] : x[0]);
            };
            // softmax and dS of element r of block blk (row 32 blk + acc_row(r, hi))
            float pv[16], dsv[16];
            auto soft = [&](int blk, int r) {
                const int g = r >> 2, i = r & 3;
                float p = fast_exp2(fmaf(sacc[r], cl2, -lc[g][i]));
                if (MASK)
                    p = ((!CAUSAL || 32 * blk + 8 * g + i >= mlim) && (!BLOCKMASK || ((allow >> blk) & 1u)))
                            ? p
                            : 0.f;
                if constexpr (DROP) {
                    const bool keep = drop_keep(md[g], i, dp.t8);
                    pv[r] = keep ? p * dp.scale : 0.f;
                    dsv[r] = p * ((keep ? dpacc[r] * dp.scale : 0.f) - dc[g][i]);
                } else {
                    pv[r] = p;
                    dsv[r] = p * (dpacc[r] - dc[g][i]);
                }
                if (r & 1) {
                    const int par = blk & 1;
                    pb[par][r >> 3][(r & 7) >> 1] = Mma<T>::pack2(pv[r - 1], pv[r]);
                    dsb[par][r >> 3][(r & 7) >> 1] = Mma<T>::pack2(dsv[r - 1], dsv[r]);
                }
            };

#pragma unroll
            for (int k = 0; k < 8; ++k) load_rows(0, k);
            if constexpr (DROP)
#pragma unroll
                for (int g = 0; g < 4; ++g) load_drop(0, g);
            static_for<AHEAD>([&](auto nc) { load_op(nc); });
            static_for<TSLOT>([&](auto nc) {
                constexpr int n = decltype(nc)::value;
                constexpr int seg = n / NSLOT, j = n % NSLOT;
                constexpr bool is_s = dkdv_seg_is_s<NQB>(seg);
                constexpr int blk = dkdv_seg_block<NQB>(seg);
                if constexpr (n == NSLOT) {
                    // block 0's softmax has no matrix work to overlap with
#pragma unroll
                    for (int r = 0; r < 16; ++r) soft(0, r);
                    __builtin_amdgcn_sched_barrier(0);
                }
                if constexpr (n + AHEAD < TSLOT) load_op(std::integral_constant<int, n + AHEAD>{});
                if constexpr (is_s) {
                    constexpr int ks = j >> 1;
                    if constexpr (j & 1)
                        dpacc = Mma<T>::mma(op[n], vf[ks], ks == 0 ? zero16() : dpacc);
                    else
                        sacc = Mma<T>::mma(op[n], kf[ks], ks == 0 ? zero16() : sacc);
                    // the softmax reads S and dP with vector instructions
                    if constexpr (j == NSLOT - 2) asm volatile("" : "+v"(sacc));
                    if constexpr (j == NSLOT - 1) asm volatile("" : "+v"(dpacc));
                } else {
                    constexpr int t = j / (2 * NDB), db = (j >> 1) % NDB;
                    constexpr int par = blk & 1;
                    if constexpr (j & 1)
                        dkt[db] = Mma<T>::mma(op[n], dsb[par][t], dkt[db]);
                    else
                        dvt[db] = Mma<T>::mma(op[n], pb[par][t], dvt[db]);
                }
                if constexpr (!is_s && seg < NSEG - 1) {
                    // a dV/dK segment of block seg/2 - 1 carries the softmax of block seg/2
#pragma unroll
                    for (int e = 0; e < EPS; ++e) soft(seg / 2, j * EPS + e);
                } else if constexpr (is_s && seg > 0 && j >= NSLOT - 8) {
                    // row terms of the block whose S/dP this segment computes
                    load_rows(blk, j - (NSLOT - 8));
                }
                // keep bytes of the block whose S/dP this segment computes
                if constexpr (DROP && is_s && seg > 0 && j < 4) load_drop(blk, j);
                if constexpr (DROP && seg == NSEG - 1) {
                    // the rounds of the next step's generator calls, spread over
                    // the last segment (it carries no softmax work)
#pragma unroll
                    for (int ri = j * NROUND / NSLOT; ri < (j + 1) * NROUND / NSLOT; ++ri) pg[ri % NCALL].round();
                }
                __builtin_amdgcn_sched_barrier(0);
            });
            // this step's byte reads are all issued, and the wave's LDS
            // operations run in order: the next step's bytes can replace them
            drop_store(dr);
        };

        if (!BLOCKMASK && nsteps > 0) {
            issue(0, buf_of(0));
            put_rows(buf_of(0));
            if constexpr (DROP) {
                drop_start(0);
#pragma unroll
                for (int r = 0; r < 10; ++r)
#pragma unroll
                    for (int c = 0; c < NCALL; ++c) pg[c].round();
                drop_store(dbase);
            }
        }
        wait_vmem();
        __syncthreads();
        read_kv();
        __syncthreads();   // every wave holds its K/V before the next step's copies

        // one tile: prefetch the next one into the other buffer, compute, publish
        auto tile = [&](int s, auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
            constexpr int BUFC = decltype(buf_tag)::value;
            const int nb = buf_of(s) ^ 1;
            issue(min(s + 1, nsteps - 1), nb);
            int h, q0;
            step_rows(s, h, q0);
            (void)h;
            // rows q0 + 4 hi + (32 blk + 8 g + i) are visible when at or after the key
            run_step(mask_tag, smem + (BUFC >= 0 ? BUFC : buf_of(s)) * STAGE, key - q0 - 4 * hi, ~0u,
                     min(s + 1, nsteps - 1), dbase);
            put_rows(nb);
            wait_vmem();
            __syncthreads();
        };
        if constexpr (!BLOCKMASK) {
            for (int s = 0; s < ndiag; ++s)
                tile(s, std::true_type{}, std::integral_constant<int, -1>{});
            for (int s = ndiag; s < nsteps; s += 2) {
                tile(s, std::false_type{}, std::integral_constant<int, 0>{});
                if (s + 1 < nsteps) tile(s + 1, std::false_type{}, std::integral_constant<int, 1>{});
            }
        } else {
            // allow bit blk: the mask block of query rows q0 + 32 blk .. and
            // this workgroup's keys is set
            const int mc = min(kv0 / 128, sp.nb - 1);
            auto allow_of = [&](int st) {
                int h, q0;
                step_rows(st, h, q0);
                const unsigned char* col = sp.mask + (size_t)(sp.heads == 1 ? 0 : h) * sp.nb * sp.nb + mc;
                uint32_t m = 0;
#pragma unroll
                for (int r = 0; r < BQ / 128; ++r)
                    if (col[(size_t)min(q0 / 128 + r, sp.nb - 1) * sp.nb]) m |= ((1u << 4) - 1) << (4 * r);
                return m;
            };
            // The next step with a set bit, and its bits.  Each lane of the wave
            // tests one candidate (scan_load fetches its bits), so a scan costs
            // one load latency per 64 steps; scan_pick takes the first hit, or
            // loads the next 64 candidates.  The walk loads the candidates
            // after the next step before running the current one, so their
            // latency hides behind its matrix work.
            int cbase = 0;
            uint32_t cand = 0;
            auto scan_load = [&](int after) {
                cbase = after + 1;
                cand = cbase + lane < nsteps ? allow_of(cbase + lane) : 0u;
            };
            auto scan_pick = [&](uint32_t& m) {
                for (;;) {
                    const uint64_t bal = __ballot(cand != 0);
                    if (bal) {
                        const int f = __builtin_ctzll(bal);
                        m = (uint32_t)__builtin_amdgcn_readlane((int)cand, f);
                        return cbase + f;
                    }
                    if (cbase + 64 >= nsteps) break;
                    scan_load(cbase + 63);
                }
                m = 0;
                return nsteps;
            };
            // the allowed steps in the order above, buffers alternating from 0
            uint32_t m = 0, mn = 0;
            scan_load(-1);
            int s = scan_pick(m);
            if (s < nsteps) {
                issue(s, 0);
                put_rows(0);
                wait_vmem();
            }
            __syncthreads();
            int sn = nsteps;
            if (s < nsteps) {
                scan_load(s);
                sn = scan_pick(mn);
            }
            for (int par = 0; s < nsteps; par ^= 1) {
                // past the last allowed step, re-copy a valid step into the
                // buffer nobody reads again
                issue(min(sn, nsteps - 1), par ^ 1);
                if (sn < nsteps) scan_load(sn);
                int h, q0;
                step_rows(s, h, q0);
                (void)h;
                run_step(std::true_type{}, smem + par * STAGE, key - q0 - 4 * hi, m, 0, dbase);
                put_rows(par ^ 1);
                uint32_t mnn = 0;
                const int snn = sn < nsteps ? scan_pick(mnn) : nsteps;
                wait_vmem();
                __syncthreads();
                s = sn;
                m = mn;
                sn = snn;
                mn = mnn;
            }
        }

        {
            // dK and dV rows go through this wave's own 16 KB of buffer 0 (free
            // after the walk's last barrier): each lane writes its 8-byte pieces
            // in the swizzled layout, then reads back 16-byte chunks in row
            // order, so that each store writes 1 KB of consecutive rows.  Keys
            // past the sequence's length (their columns of dS and P need not be
            // finite) get zero gradients.  A barrier ends the block, so that no
            // wave copies the next block's first step over rows another wave is
            // still reading back.
            int ln = lane;
            asm volatile("" : "+v"(ln));
            unsigned char* const ost = smem + wave * (2 * 32 * D * 2);
            const bool pad = SPARSE && kw + (ln & 31) >= Nk;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    u32x2 wk, wv;
                    wk[0] = Mma<T>::pack2(dkt[db][4 * g] * scale, dkt[db][4 * g + 1] * scale);
                    wk[1] = Mma<T>::pack2(dkt[db][4 * g + 2] * scale, dkt[db][4 * g + 3] * scale);
                    wv[0] = Mma<T>::pack2(dvt[db][4 * g], dvt[db][4 * g + 1]);
                    wv[1] = Mma<T>::pack2(dvt[db][4 * g + 2], dvt[db][4 * g + 3]);
                    if (pad) wk = wv = u32x2{0u, 0u};
                    const int o = kq_off<D>(ln & 31, 4 * db + g) + 8 * (ln >> 5);
                    *reinterpret_cast<u32x2*>(ost + o) = wk;
                    *reinterpret_cast<u32x2*>(ost + 32 * D * 2 + o) = wv;
                }
            unsigned char* const dkw = reinterpret_cast<unsigned char*>(dK + kvoff + (size_t)kw * D);
            unsigned char* const dvw = reinterpret_cast<unsigned char*>(dV + kvoff + (size_t)kw * D);
#pragma unroll
            for (int k = 0; k < 32 / KRPC; ++k) {
                const int r = KRPC * k + ln / KCH;
                const int o = kq_off<D>(r, ln % KCH);
                const u32x4 vk = *reinterpret_cast<const u32x4*>(ost + o);
                const u32x4 vv = *reinterpret_cast<const u32x4*>(ost + 32 * D * 2 + o);
                if (kw + r < N) {
                    *reinterpret_cast<u32x4*>(dkw + 1024 * k + 16 * ln) = vk;
                    *reinterpret_cast<u32x4*>(dvw + 1024 * k + 16 * ln) = vv;
                }
            }
            __syncthreads();
        }

    }
    FA355_CLOCK_END(fa355_clock_bwd)
}

// ---------------------------------------------------------------------------
// Third-generation dQ kernel, query-outer: a workgroup holds 32 NW query rows
// (Q and dO in registers, one row per lane) and walks the key tiles, which
// arrive by buffer-to-LDS copies, row-major only; the K^T operands of
// dQ^T += K^T dS^T come from transposing reads of the same K tile (dual
// swizzle), so no transposed copy is built.  The key tiles are split in two
// loops.  Tiles wholly below every row of the block (and inside the sequence)
// run a body with no mask code, two at a time so that both LDS buffers have
// compile-time offsets; the diagonal and ragged-end tiles run the masked body.
//
// DROP: attention dropout (fa_common.h): dS = P * (Z dP 256 / t8 - D), with
// the keep bytes of a tile's key blocks drawn as in the forward kernel (lane
// half hi draws block 2 kp + hi of its row, one exchange per block pair).
//
// SPARSE: variable lengths and block masks.  Keys past the sequence's length
// read as zeros and are masked like a ragged end; a row past it, or a row with
// no visible key (logsumexp -inf), takes an infinite logsumexp, so its P and
// dS are exactly zero on every tile.  With a block mask the workgroup's 128
// rows are one mask row and the walk visits only the key tiles it allows.
template <typename T, int D, bool CAUSAL, int NW = 4, bool DROP = false, bool SPARSE = false>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
dq16v3_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
              const uint16_t* __restrict__ V, const uint16_t* __restrict__ dO,
              const float* __restrict__ LSE, const float* __restrict__ Delta,
              uint16_t* __restrict__ dQ, int B, int Hq, int Hkv, int N, float cl2, float scale,
              DropParams dp, SparseParams sp) {
    FA355_CLOCK_BEGIN
    static_assert(!SPARSE || NW == 4, "a block-mask row spans the workgroup's 128 rows");
    constexpr int BR = 32 * NW;
    constexpr int BC = D == 128 ? FA355_DQ_BC128 : 128;
    constexpr int KCH = D / 8;
    constexpr int TB = BC * D * 2;
    constexpr int STAGE = 2 * TB;
    constexpr int NKB = BC / 32;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr int WI = TB / 1024;
    static_assert(WI % NW == 0, "tile copies split evenly over the waves");
    constexpr int IPW = WI / NW;

    __shared__ __attribute__((aligned(16))) unsigned char smem[2 * STAGE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int nqb = (N + BR - 1) / BR;
    const int total = nqb * Hq * B;
    const int logical = xcd_remap((int)blockIdx.x, total);
    const int qb_raw = logical % nqb;
    const int bh = logical / nqb;
    const int qb = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;
    // the masked path takes the batch index fastest (XCD balance across
    // sequences of different lengths)
    const int h = SPARSE ? bh / B : bh % Hq;
    const int b = SPARSE ? bh % B : bh / Hq;
    const int hk = h / (Hq / Hkv);

    const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
    const size_t koff = ((size_t)b * Hkv + hk) * (size_t)N * D;
    // valid positions of this sequence (the masked path's lengths; else N)
    const int Nk = (SPARSE && sp.seqlens) ? min(max(sp.seqlens[b], 0), N) : N;
    const uint32_t head_bytes = (uint32_t)N * D * 2;
    const Buf Kb(K + koff, (uint32_t)Nk * D * 2), Vb(V + koff, (uint32_t)Nk * D * 2);

    const int q0 = qb * BR;
    const int qw = q0 + 32 * wave;
    const int q = qw + l32;

    u32x4 qf[NKS], dof[NKS];
    {
        const Buf Qb(Q + qoff, head_bytes), Db(dO + qoff, head_bytes);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            qf[ks] = Qb.load16((uint32_t)(q * D + 16 * ks + 8 * hi) * 2);
            dof[ks] = Db.load16((uint32_t)(q * D + 16 * ks + 8 * hi) * 2);
        }
    }
    const size_t roff = ((size_t)b * Hq + h) * (size_t)N;
    float lse2 = Buf(LSE + roff, (uint32_t)N * 4).load_f32((uint32_t)q * 4) * kLog2e;
    const float dlt = Buf(Delta + roff, (uint32_t)N * 4).load_f32((uint32_t)q * 4);
    // padded and empty rows: P = exp2(S - inf) = 0 everywhere
    if (SPARSE && (q >= Nk || !(lse2 > -INFINITY))) lse2 = INFINITY;

    const int kv_len = (SPARSE && q0 >= Nk) ? 0 : (CAUSAL ? min(Nk, q0 + BR) : Nk);
    const int ntiles = (kv_len + BC - 1) / BC;

    uint32_t cp[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int p = (wave + NW * i) * 64 + lane;
        const int row = p / KCH, pc = p % KCH;
        cp[i] = (uint32_t)(row * D * 2 + 16 * (pc ^ dual_swz<D>(row)));
    }
    auto issue_to = [&](unsigned char* base, int k0) {
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const uint32_t off = (uint32_t)k0 * D * 2 + cp[i];
            buf_to_lds16(Kb, base + (wave + NW * i) * 1024, off);
            buf_to_lds16(Vb, base + TB + (wave + NW * i) * 1024, off);
        }
    };

    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = 4 * hi + (j16 >> 2);
    const int tr_col = 2 * (16 * (g16 & 1) + 4 * (j16 & 3));

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = zero16();

    // Tile j from the buffer at base.  ISSUE: the copies of key tile kn go to
    // the buffer at nxt first; the two restrict-qualified buffer pointers let
    // the compiler see that the transposing reads of this tile never touch
    // what the copies write, so they do not wait for the copies in flight.
    auto body = [&](int j, auto mask_tag, auto issue_tag, const unsigned char* __restrict__ base,
                    unsigned char* __restrict__ nxt, int kn) __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        if constexpr (decltype(issue_tag)::value) issue_to(nxt, kn);
        const int k0 = j * BC;
        uint32_t dm[DROP ? NKB : 1][4];
        if constexpr (DROP) {
#pragma unroll
            for (int kp = 0; kp < NKB / 2; ++kp) {
                uint32_t w[8];
                drop_bytes(w, (uint32_t)(k0 / 32 + 2 * kp + hi), (uint32_t)q, (uint32_t)(b * Hq + h), dp);
                drop_pair_exchange(w, dm[2 * kp], dm[2 * kp + 1]);
            }
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            f32x16 st = zero16(), dpt = zero16();
            // raised priority while the wave issues its S and dP products: when
            // both waves of a SIMD are ready, the one feeding the matrix cores
            // issues first
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                const int off = dual_off<D>(32 * kb + l32, 16 * (2 * ks + hi));
                const u32x4 ak = *reinterpret_cast<const u32x4*>(base + off);
                const u32x4 av = *reinterpret_cast<const u32x4*>(base + TB + off);
                st = Mma<T>::mma(ak, qf[ks], st);
                dpt = Mma<T>::mma(av, dof[ks], dpt);
            }
            __builtin_amdgcn_s_setprio(0);
            float p[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) p[r] = fast_exp2(fmaf(st[r], cl2, -lse2));
            if (MASK) {
                // key k0 + 32 kb + acc_row(r, hi) is visible iff it is at most
                // min(q, Nk - 1) (Nk - 1 without the causal mask): one compare of
                // the register's constant part against a per-lane limit
                const int lim = (CAUSAL ? min(q, Nk - 1) : Nk - 1) - (k0 + 32 * kb) - 4 * hi;
#pragma unroll
                for (int r = 0; r < 16; ++r) p[r] = (8 * (r >> 2) + (r & 3) <= lim) ? p[r] : 0.f;
            }
            if constexpr (DROP) {
                // register r: byte r % 4 of dword r / 4
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    dpt[r] = drop_keep(dm[kb][r >> 2], r & 3, dp.t8) ? dpt[r] * dp.scale : 0.f;
            }
            u32x4 dsb[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const int r = 8 * t + 2 * jj;
                    dsb[t][jj] = Mma<T>::pack2(p[r] * (dpt[r] - dlt), p[r + 1] * (dpt[r + 1] - dlt));
                }
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const int row = 32 * kb + 16 * t + tr_row;
                    const int col = 64 * db + tr_col;
                    const u32x2 lo = lds_read_tr16(base + dual_off<D>(row, col));
                    const u32x2 up = lds_read_tr16(base + dual_off<D>(row + 8, col));
                    u32x4 a;
                    a[0] = lo[0]; a[1] = lo[1]; a[2] = up[0]; a[3] = up[1];
                    dq[db] = Mma<T>::mma(a, dsb[t], dq[db]);
                }
        }
    };

    // tiles below every row of the block and inside the sequence
    const int nfull = min(min(CAUSAL ? q0 / BC : ntiles, Nk / BC), ntiles);
    // The copy of the next tile is issued at the start of every tile, also the
    // last (it lies in this head's range or past its end and reads as zeros).
    if constexpr (!SPARSE) {
        issue_to(smem, 0);
        wait_vmem();
        __syncthreads();
        int j = 0;
        for (; j + 1 < nfull; j += 2) {
            body(j, std::false_type{}, std::true_type{}, smem, smem + STAGE, (j + 1) * BC);
            wait_vmem();
            __syncthreads();
            body(j + 1, std::false_type{}, std::true_type{}, smem + STAGE, smem, (j + 2) * BC);
            wait_vmem();
            __syncthreads();
        }
        for (; j < ntiles; ++j) {
            issue_to(smem + ((j + 1) & 1) * STAGE, (j + 1) * BC);
            if (!CAUSAL || j * BC <= qw + 31)
                body(j, std::true_type{}, std::false_type{}, smem + (j & 1) * STAGE, nullptr, 0);
            wait_vmem();
            __syncthreads();
        }
    } else {
        // the same walk over the key tiles the block mask allows for this row
        // block (all of them without one)
        const unsigned char* mrow =
            sp.mask ? sp.mask + ((size_t)(sp.heads == 1 ? 0 : h) * sp.nb + min(q0 / 128, sp.nb - 1)) * sp.nb
                    : nullptr;
        // the next allowed tile after jt: each lane of the wave tests one
        // candidate, so a scan costs one load latency per 64 tiles
        auto next = [&](int jt) {
            if (!mrow) return jt + 1;
            for (int base = jt + 1; base < ntiles; base += 64) {
                const int c = base + lane;
                const uint64_t bal = __ballot(c < ntiles && mrow[c * BC / 128] != 0);
                if (bal) return base + __builtin_ctzll(bal);
            }
            return ntiles;
        };
        int j = next(-1);
        issue_to(smem, j * BC);
        wait_vmem();
        __syncthreads();
        for (;;) {
            const int j1 = next(j);
            if (j1 >= nfull) break;
            const int j2 = next(j1);
            body(j, std::false_type{}, std::true_type{}, smem, smem + STAGE, j1 * BC);
            wait_vmem();
            __syncthreads();
            body(j1, std::false_type{}, std::true_type{}, smem + STAGE, smem, j2 * BC);
            wait_vmem();
            __syncthreads();
            j = j2;
        }
        for (int par = 0; j < ntiles; par ^= 1) {
            const int jn = next(j);
            issue_to(smem + (par ^ 1) * STAGE, jn * BC);
            if (!CAUSAL || j * BC <= qw + 31)
                body(j, std::true_type{}, std::false_type{}, smem + par * STAGE, nullptr, 0);
            wait_vmem();
            __syncthreads();
            j = jn;
        }
    }

    {
        // dQ rows go through LDS (free after the walk's last barrier): each lane
        // writes its 8-byte pieces in the swizzled layout, then reads back
        // 16-byte chunks in row order, so that each store writes 1 KB of
        // consecutive rows instead of 8 bytes in each of 32 rows.  (The lane
        // index goes through an empty asm, so that the staging addresses are
        // formed here rather than held through the walk.)
        static_assert(NW * 32 * D * 2 <= 2 * STAGE, "dQ staging fits the K/V buffers");
        constexpr int RPC = 1024 / (D * 2);   // rows per 1 KB store
        int ln = lane;
        asm volatile("" : "+v"(ln));
        unsigned char* const ost = smem + wave * (32 * D * 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = Mma<T>::pack2(dq[db][4 * g] * scale, dq[db][4 * g + 1] * scale);
                w[1] = Mma<T>::pack2(dq[db][4 * g + 2] * scale, dq[db][4 * g + 3] * scale);
                *reinterpret_cast<u32x2*>(ost + kq_off<D>(ln & 31, 4 * db + g) + 8 * (ln >> 5)) = w;
            }
        unsigned char* const dqw = reinterpret_cast<unsigned char*>(dQ + qoff + (size_t)qw * D);
#pragma unroll
        for (int k = 0; k < 32 / RPC; ++k) {
            const int r = RPC * k + ln / KCH;
            const u32x4 v = *reinterpret_cast<const u32x4*>(ost + kq_off<D>(r, ln % KCH));
            if (qw + r < N) *reinterpret_cast<u32x4*>(dqw + 1024 * k + 16 * ln) = v;
        }
    }
    FA355_CLOCK_END(fa355_clock_bwd)
}

// ---------------------------------------------------------------------------
// fp32 inputs: the same two passes with the fp32 matrix-core op (32x32x2), P
// and dS kept in fp32, single-buffered LDS tiles with padded rows.
template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
dkdv32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
              const float* __restrict__ dO, const float* __restrict__ LSE,
              const float* __restrict__ Delta, float* __restrict__ dK, float* __restrict__ dV,
              int B, int Hq, int Hkv, int N, float cl2, float scale) {
    constexpr int BKV = 128;
    constexpr int BQ = 32;
    constexpr int RS = D + 1;
    constexpr int NDB = D / 32;
    __shared__ float Qs[BQ * RS];
    __shared__ float dOs[BQ * RS];
    __shared__ float lse2s[BQ];
    __shared__ float dls[BQ];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // provably wave-uniform
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int nkb = (N + BKV - 1) / BKV;
    const int total = nkb * Hkv * B;
    const int logical = xcd_remap((int)blockIdx.x, total);
    const int jb = logical % nkb;
    const int bhk = logical / nkb;
    const int hk = bhk % Hkv;
    const int b = bhk / Hkv;
    const int G = Hq / Hkv;
    const int kv0 = jb * BKV;
    const int kw = kv0 + 32 * wave;
    const int key = kw + l32;
    const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)N * D;

    float kf[D / 2], vf[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) {
        kf[ks] = key < N ? K[kvoff + (size_t)key * D + 2 * ks + hi] : 0.f;
        vf[ks] = key < N ? V[kvoff + (size_t)key * D + 2 * ks + hi] : 0.f;
    }
    f32x16 dkt[NDB], dvt[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        dkt[db] = zero16();
        dvt[db] = zero16();
    }

    const int qb_first = CAUSAL ? kv0 / BQ : 0;
    const int nqb = (N + BQ - 1) / BQ;
    for (int g = 0; g < G; ++g) {
        const int h = hk * G + g;
        const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
        const size_t roff = ((size_t)b * Hq + h) * (size_t)N;
        for (int qb = qb_first; qb < nqb; ++qb) {
            const int q0 = qb * BQ;
            __syncthreads();
            for (int i = tid; i < BQ * D; i += 256) {
                const int r = i / D, c = i % D;
                const int q = q0 + r;
                Qs[r * RS + c] = q < N ? Q[qoff + (size_t)q * D + c] : 0.f;
                dOs[r * RS + c] = q < N ? dO[qoff + (size_t)q * D + c] : 0.f;
            }
            if (tid < BQ) {
                const int q = q0 + tid;
                lse2s[tid] = q < N ? LSE[roff + q] * kLog2e : 0.f;
                dls[tid] = q < N ? Delta[roff + q] : 0.f;
            }
            __syncthreads();
            if (CAUSAL && q0 + BQ - 1 < kw) continue;

            f32x16 sacc = zero16(), dpacc = zero16();
#pragma unroll 8
            for (int ks = 0; ks < D / 2; ++ks) {
                sacc = mma_f32(Qs[l32 * RS + 2 * ks + hi], kf[ks], sacc);
                dpacc = mma_f32(dOs[l32 * RS + 2 * ks + hi], vf[ks], dpacc);
            }
            float p[16], ds[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = acc_row(r, hi);
                const int q = q0 + qr;
                const bool vis = (!CAUSAL || key <= q) && q < N && key < N;
                p[r] = vis ? fast_exp2(fmaf(sacc[r], cl2, -lse2s[qr])) : 0.f;
                ds[r] = p[r] * (dpacc[r] - dls[qr]);
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int qr = acc_row(r, hi);
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    dvt[db] = mma_f32(dOs[qr * RS + 32 * db + l32], p[r], dvt[db]);
                    dkt[db] = mma_f32(Qs[qr * RS + 32 * db + l32], ds[r], dkt[db]);
                }
            }
        }
    }

    if (key < N) {
        float* dkrow = dK + kvoff + (size_t)key * D;
        float* dvrow = dV + kvoff + (size_t)key * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 wk, wv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    wk[i] = dkt[db][4 * g + i] * scale;
                    wv[i] = dvt[db][4 * g + i];
                }
                *reinterpret_cast<f32x4*>(dkrow + 32 * db + 8 * g + 4 * hi) = wk;
                *reinterpret_cast<f32x4*>(dvrow + 32 * db + 8 * g + 4 * hi) = wv;
            }
    }
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256)
dq32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
            const float* __restrict__ dO, const float* __restrict__ LSE,
            const float* __restrict__ Delta, float* __restrict__ dQ, int B, int Hq, int Hkv, int N,
            float cl2, float scale) {
    constexpr int NW = 4;
    constexpr int BR = 32 * NW;
    constexpr int BC = 32;
    constexpr int RS = D + 1;
    constexpr int NDB = D / 32;
    __shared__ float Ks[BC * RS];
    __shared__ float Vs[BC * RS];

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

    float qf[D / 2], dof[D / 2];
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) {
        qf[ks] = q < N ? Q[qoff + (size_t)q * D + 2 * ks + hi] : 0.f;
        dof[ks] = q < N ? dO[qoff + (size_t)q * D + 2 * ks + hi] : 0.f;
    }
    const size_t roff = ((size_t)b * Hq + h) * (size_t)N;
    const float lse2 = q < N ? LSE[roff + q] * kLog2e : 0.f;
    const float dlt = q < N ? Delta[roff + q] : 0.f;

    f32x16 dq[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dq[db] = zero16();

    const int kv_len = CAUSAL ? min(N, q0 + BR) : N;
    for (int k0 = 0; k0 < kv_len; k0 += BC) {
        __syncthreads();
        for (int i = tid; i < BC * D; i += 256) {
            const int r = i / D, c = i % D;
            const int kk = k0 + r;
            Ks[r * RS + c] = kk < N ? K[koff + (size_t)kk * D + c] : 0.f;
            Vs[r * RS + c] = kk < N ? V[koff + (size_t)kk * D + c] : 0.f;
        }
        __syncthreads();
        if (CAUSAL && k0 > qw + 31) continue;

        f32x16 st = zero16(), dpt = zero16();
#pragma unroll 8
        for (int ks = 0; ks < D / 2; ++ks) {
            st = mma_f32(Ks[l32 * RS + 2 * ks + hi], qf[ks], st);
            dpt = mma_f32(Vs[l32 * RS + 2 * ks + hi], dof[ks], dpt);
        }
        float ds[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int kk = k0 + acc_row(r, hi);
            const bool vis = (!CAUSAL || kk <= q) && kk < N;
            const float p = vis ? fast_exp2(fmaf(st[r], cl2, -lse2)) : 0.f;
            ds[r] = p * (dpt[r] - dlt);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                dq[db] = mma_f32(Ks[acc_row(r, hi) * RS + 32 * db + l32], ds[r], dq[db]);
    }

    if (q < N) {
        float* row = dQ + qoff + (size_t)q * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = dq[db][4 * g + i] * scale;
                *reinterpret_cast<f32x4*>(row + 32 * db + 8 * g + 4 * hi) = w;
            }
    }
}

// ---------------------------------------------------------------------------
template <typename T, int D>
hipError_t prepare16(const BwdArgs& a) {
    const long long rows = (long long)a.B * a.Hq * a.N;
    constexpr int RPB = 256 / (D / 8);
    hipLaunchKernelGGL((delta16_kernel<T, D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       a.stream, (const uint16_t*)a.o, (const uint16_t*)a.dout, a.delta, rows);
    return hipGetLastError();
}

template <int D>
hipError_t prepare32(const BwdArgs& a) {
    const long long rows = (long long)a.B * a.Hq * a.N;
    constexpr int RPB = 256 / (D / 4);
    hipLaunchKernelGGL((delta32_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0,
                       a.stream, (const float*)a.o, (const float*)a.dout, a.delta, rows);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL>
hipError_t dkdv16(const BwdArgs& a) {
    const int nkb = (a.N + 127) / 128;
    const long long total = (long long)nkb * a.Hkv * a.B;
    // persistent grid where the key blocks outnumber the compute units; the
    // masked path keeps one workgroup per key block, since its steps per key
    // block vary with the lengths and the mask, and a static schedule would
    // leave the compute units unevenly loaded
    const int grid = persistent_grid();
    const bool pers = !a.sparse && grid >= 8 && total > grid;
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3((unsigned)(pers ? grid : total)), dim3(256), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dk, (uint16_t*)a.dv, a.B,
                           a.Hq, a.Hkv, a.N, a.cl2, a.scale, a.dp, a.sp, pers ? dkdv_pool_slot() : nullptr);
        return hipGetLastError();
    };
    if (a.sparse)
        return a.sp.mask ? go(dkdv16v3_kernel<T, D, CAUSAL, false, 2>) : go(dkdv16v3_kernel<T, D, CAUSAL, false, 1>);
    if (a.drop)
        return pers ? go(dkdv16v3_kernel<T, D, CAUSAL, true, 0, true>) : go(dkdv16v3_kernel<T, D, CAUSAL, false, 0, true>);
    return pers ? go(dkdv16v3_kernel<T, D, CAUSAL, true>) : go(dkdv16v3_kernel<T, D, CAUSAL>);
}

template <typename T, int D, bool CAUSAL>
hipError_t dq16(const BwdArgs& a) {
    auto go = [&](auto kern) {
        // kern's rows per workgroup: 32 per wave (dense path: FA355_DQ_NW waves)
        const int nw = (a.sparse || a.drop) ? 4 : FA355_DQ_NW;
        const int nqb = (a.N + 32 * nw - 1) / (32 * nw);
        hipLaunchKernelGGL(kern, dim3((unsigned)(nqb * a.Hq * a.B)), dim3(64 * nw), 0, a.stream,
                           (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                           (const uint16_t*)a.dout, a.lse, a.delta, (uint16_t*)a.dq, a.B, a.Hq, a.Hkv,
                           a.N, a.cl2, a.scale, a.dp, a.sp);
        return hipGetLastError();
    };
    if (a.sparse) return go(dq16v3_kernel<T, D, CAUSAL, 4, false, true>);
    if (a.drop) return go(dq16v3_kernel<T, D, CAUSAL, 4, true>);
    return go(dq16v3_kernel<T, D, CAUSAL, FA355_DQ_NW>);
}

template <int D, bool CAUSAL>
hipError_t dkdv32(const BwdArgs& a) {
    const int nkb = (a.N + 127) / 128;
    hipLaunchKernelGGL((dkdv32_kernel<D, CAUSAL>), dim3((unsigned)(nkb * a.Hkv * a.B)), dim3(256), 0,
                       a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dout, a.lse, a.delta, (float*)a.dk, (float*)a.dv, a.B, a.Hq,
                       a.Hkv, a.N, a.cl2, a.scale);
    return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t dq32(const BwdArgs& a) {
    const int nqb = (a.N + 127) / 128;
    hipLaunchKernelGGL((dq32_kernel<D, CAUSAL>), dim3((unsigned)(nqb * a.Hq * a.B)), dim3(256), 0,
                       a.stream, (const float*)a.q, (const float*)a.k, (const float*)a.v,
                       (const float*)a.dout, a.lse, a.delta, (float*)a.dq, a.B, a.Hq, a.Hkv, a.N,
                       a.cl2, a.scale);
    return hipGetLastError();
}

// dtype x head dim x mask -> instance.
template <template <typename, int, bool> class F16, template <int, bool> class F32>
hipError_t pick(const BwdArgs& a) {
    const bool c = a.causal != 0;
    switch (a.dtype) {
        case 2:
            return a.d == 64 ? (c ? F16<BF16, 64, true>::run(a) : F16<BF16, 64, false>::run(a))
                             : (c ? F16<BF16, 128, true>::run(a) : F16<BF16, 128, false>::run(a));
        case 1:
            return a.d == 64 ? (c ? F16<FP16, 64, true>::run(a) : F16<FP16, 64, false>::run(a))
                             : (c ? F16<FP16, 128, true>::run(a) : F16<FP16, 128, false>::run(a));
        default:
            return a.d == 64 ? (c ? F32<64, true>::run(a) : F32<64, false>::run(a))
                             : (c ? F32<128, true>::run(a) : F32<128, false>::run(a));
    }
}

template <typename T, int D, bool C> struct Dkdv16 { static hipError_t run(const BwdArgs& a) { return dkdv16<T, D, C>(a); } };
template <int D, bool C> struct Dkdv32 { static hipError_t run(const BwdArgs& a) { return dkdv32<D, C>(a); } };
template <typename T, int D, bool C> struct Dq16 { static hipError_t run(const BwdArgs& a) { return dq16<T, D, C>(a); } };
template <int D, bool C> struct Dq32 { static hipError_t run(const BwdArgs& a) { return dq32<D, C>(a); } };

}  // namespace

hipError_t launch_bwd_prepare(const BwdArgs& a) {
    switch (a.dtype) {
        case 2: return a.d == 64 ? prepare16<BF16, 64>(a) : prepare16<BF16, 128>(a);
        case 1: return a.d == 64 ? prepare16<FP16, 64>(a) : prepare16<FP16, 128>(a);
        default: return a.d == 64 ? prepare32<64>(a) : prepare32<128>(a);
    }
}

hipError_t launch_bwd_dkdv(const BwdArgs& a) { return pick<Dkdv16, Dkdv32>(a); }

hipError_t launch_bwd_dq(const BwdArgs& a) { return pick<Dq16, Dq32>(a); }

}  // namespace fa355
