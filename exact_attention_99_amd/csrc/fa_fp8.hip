// FP8 forward path: the block quantizer and the e4m3 attention kernel.
//
// Low-precision attention with block quantization and a rotation that
// spreads outlier features ("FlashAttention 1, 2, and 3 Explained",
// section 4 on FlashAttention-3: FP8 with block quantization and incoherent
// processing; "FlashAttention" glossary, FlashAttention-3 paragraph):
//
//   quantize: x [N, d] per head -> optional rotation y = (x * s) H / sqrt(d)
//             (fast Walsh-Hadamard transform, the same signs s for Q and K so
//             that every score q . k is unchanged), then per block of 64 rows
//             scale = amax / 448 and codes = e4m3(y * 448 / amax).
//   forward:  exact attention of the dequantized values, with both products
//             on the e4m3 matrix cores (v_mfma_scale_f32_32x32x64_f8f6f4,
//             2x the 16-bit rate) and the probabilities rounded to e4m3 for
//             the P V product.
//
// e4m3 operand layout of the 32x32x64 product (one 64-lane wave, l32 = l %
// 32, hi = l / 32): lane l holds A[l32][32 hi .. 32 hi + 31] and
// B[32 hi .. 32 hi + 31][l32] (32 bytes each); D as for the 16-bit products.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa355 {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kQBlk = 64;          // rows per quantization block
constexpr float kE4m3Max = 448.f;  // largest finite e4m3 value
// The probabilities enter the P V product as e4m3 values 2^(x - m + kPOff)
// (m = running row maximum): the shift moves the largest ones to the top of
// the e4m3 range, where its 3 mantissa bits are normal numbers.  The running
// maximum moves once a tile's maximum exceeds it by more than kTau8, so every
// value stays below 2^(kPOff + kTau8) < 448.
constexpr float kPOff = 8.f;
constexpr float kTau8 = 0.75f;

__device__ __forceinline__ f32x16 mma8(i32x8 a, i32x8 b, f32x16 c) {
    // operand formats 0 (e4m3) for A and B; block scales 2^0 (E8M0 127)
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(u32x4 a, u32x4 b) {
    i32x8 r;
    r[0] = (int)a[0]; r[1] = (int)a[1]; r[2] = (int)a[2]; r[3] = (int)a[3];
    r[4] = (int)b[0]; r[5] = (int)b[1]; r[6] = (int)b[2]; r[7] = (int)b[3];
    return r;
}

// Transposing 8-bit LDS read (ds_read_b64_tr_b8): within each group of 16
// lanes, when lane s addresses row r0 + s / 2, bytes c0 + 8 (s % 2) .. +7 of
// a row-major byte tile, lane i receives column c0 + i of rows r0 .. r0 + 7.
__device__ __forceinline__ i32x2 lds_read_tr8(const void* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) i32x2*)(p));
}

// Four fp32 values -> one dword of e4m3 codes (round to nearest even; the
// inputs are within +-448).
__device__ __forceinline__ int pack4_e4m3(float a, float b, float c, float d) {
    // the first conversion's upper half is overwritten by the second, so its
    // "old" operand is a don't-care (a's register; no zeroing move)
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// ---------------------------------------------------------------- quantizer

// XOR swizzles of the quantizer's LDS tiles (16-byte chunks): chunk k of row
// r sits in slot k ^ sw(r) of that row, so that the 8 or 16 lanes of one
// 128-bit LDS access (one row each, or one row's chunks) fall on distinct
// banks.
template <int D>
__device__ __forceinline__ int qin_sw(int r) {   // input rows: 2 D bytes
    return D == 128 ? (r & 15) : ((r & 7) ^ ((r >> 3) & 1));
}
template <int D>
__device__ __forceinline__ int qout_sw(int r) {  // code rows: D bytes
    return D == 128 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 1) & 3);
}

// One wave per block of 64 rows of one head; lane l holds row 64 blk + l
// whole, so every butterfly of the rotation is a pair of registers of one lane
// (no lane exchanges).  The block (contiguous in memory) comes in through
// coalesced buffer-to-LDS copies and the codes leave through coalesced stores;
// the LDS tile turns rows into lanes.  Butterflies with strides 1, 2, 4, ...,
// D / 2, then one multiplication by rs = fp32(1 / sqrt(D)).  The signs are
// wave-uniform (scalar loads); as they are +-1, the stride-1 butterfly takes
// them in exactly: (s_a a + s_b b, s_a a - s_b b) = (fma(b, s_b, t),
// fma(b, -s_b, t)) with t = s_a a, the same roundings as multiplying first.
template <typename T, int D, bool ROT>
__global__ void __launch_bounds__(64)
quant8_kernel(const uint16_t* __restrict__ X, const float* __restrict__ signs, float rs,
              uint8_t* __restrict__ C, float* __restrict__ S, int N, int nblk) {
    constexpr int RC = D / 8;     // 16-byte chunks per input row
    constexpr int RPI = 64 / RC;  // input rows per 1 KB copy
    constexpr int OC = D / 16;    // 16-byte chunks per code row
    constexpr int OPI = 64 / OC;  // code rows per 1 KB store
    __shared__ __attribute__((aligned(16))) uint8_t tile[kQBlk * D * 2];
    const int lane = threadIdx.x;
    const int blk = (int)blockIdx.x % nblk;
    const size_t head = blockIdx.x / nblk;
    const Buf xb(X + head * (size_t)N * D, (uint32_t)N * D * 2);

    // copy c: lane j brings chunk (j % RC) ^ qin_sw(row) of row RPI c + j / RC
    // to tile byte 1024 c + 16 j, which is where that chunk's slot is; rows
    // past N arrive as zeros (buffer range)
#pragma unroll
    for (int c = 0; c < kQBlk / RPI; ++c) {
        const int row = RPI * c + lane / RC;
        const int chunk = (lane % RC) ^ qin_sw<D>(row);
        buf_to_lds16(xb, tile + 1024 * c, (uint32_t)(((blk * kQBlk + row) * D + 8 * chunk) * 2));
    }
    wait_vmem();
    __syncthreads();

    float y[D];
#pragma unroll
    for (int k = 0; k < RC; ++k) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(tile + lane * 2 * D + 16 * (k ^ qin_sw<D>(lane)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            y[8 * k + 2 * i] = Mma<T>::to_f32((uint16_t)(w[i] & 0xFFFFu));
            y[8 * k + 2 * i + 1] = Mma<T>::to_f32((uint16_t)(w[i] >> 16));
        }
    }
    if (ROT) {
#pragma unroll
        for (int i = 0; i < D; i += 2) {
            const float t = y[i] * signs[i];
            const float b = y[i + 1], sb = signs[i + 1];
            y[i] = fmaf(b, sb, t);
            y[i + 1] = fmaf(b, -sb, t);
        }
#pragma unroll
        for (int h = 2; h < D; h *= 2)
#pragma unroll
            for (int i = 0; i < D; ++i)
                if ((i & h) == 0) {
                    const float a = y[i], b = y[i + h];
                    y[i] = a + b;
                    y[i + h] = a - b;
                }
#pragma unroll
        for (int i = 0; i < D; ++i) y[i] *= rs;
    }

    float mx[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < D; ++i) mx[i & 3] = fmaxf(mx[i & 3], fabsf(y[i]));
    float amax = fmaxf(fmaxf(mx[0], mx[1]), fmaxf(mx[2], mx[3]));
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    // a block whose amax is 0, or so small that 448 / amax overflows, is
    // stored as zeros with scale 1
    const float inv = kE4m3Max / amax;
    const bool flush = __builtin_amdgcn_readfirstlane(!(inv <= __FLT_MAX__) ? 1 : 0) != 0;

    // codes of row `lane` into its tile row (slots qout_sw), then out in
    // coalesced 1 KB stores (store c covers rows OPI c .. OPI c + OPI - 1),
    // non-temporal: nothing reads them back before they leave the caches.
    // No clamp to +-448 is needed: |y inv| <= amax fl(448 / amax) rounds to at
    // most 448 (1 + 2^-23)^2, and the conversion rounds to nearest before its
    // range check (values below 464 encode as 448).
    // (A flushed block's codes are formed like any other and then replaced by
    // zeros in the stores below, where none of y is live any more.)
    __syncthreads();
#pragma unroll
    for (int c = 0; c < OC; ++c) {
        u32x4 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) v[i] = y[16 * c + 4 * j + i] * inv;
            out[j] = (uint32_t)pack4_e4m3(v[0], v[1], v[2], v[3]);
        }
        *reinterpret_cast<u32x4*>(tile + lane * D + 16 * (c ^ qout_sw<D>(lane))) = out;
    }
    __syncthreads();
    uint8_t* dst = C + head * (size_t)N * D + (size_t)blk * kQBlk * D;
    const bool full = (blk + 1) * kQBlk <= N;
    auto store_rows = [&](auto zero_tag) {
#pragma unroll
        for (int c = 0; c < kQBlk / OPI; ++c) {
            const int row = OPI * c + lane / OC;
            const u32x4 v = decltype(zero_tag)::value
                                ? u32x4{0u, 0u, 0u, 0u}
                                : *reinterpret_cast<const u32x4*>(tile + row * D + 16 * ((lane % OC) ^ qout_sw<D>(row)));
            if (full || blk * kQBlk + row < N)
                __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + 1024 * c + 16 * lane));
        }
    };
    if (flush)
        store_rows(std::true_type{});
    else
        store_rows(std::false_type{});
    if (lane == 0) S[head * nblk + blk] = flush ? 1.f : amax / kE4m3Max;
}

// ------------------------------------------------------------ the forward

// LDS layouts of the byte tiles (row = key, D bytes per row, 16-byte chunks).
// K is read as the A operand: lane l32 of a 32-key block reads key row
// key_perm(l32), 32 bytes; the swizzle keeps the 16 lanes of each 128-bit
// read (rows {0..7, 16..23} or {8..15, 24..31} of the block) on distinct banks.
template <int D>
__device__ __forceinline__ int k8_swz(int r) {
    return D == 128 ? (((r >> 1) & 3) | ((r >> 2) & 4)) : (((r >> 2) & 1) | ((r >> 3) & 2));
}
// V is read through the transposing read (8 consecutive rows, 16 bytes each,
// per 16 lanes; two such groups of adjacent chunks per 32 lanes).
template <int D>
__device__ __forceinline__ int v8_swz(int r) {
    return D == 128 ? (r & 7) : (2 * ((r >> 2) & 1));
}
template <int D>
__device__ __forceinline__ int k8_off(int row, int chunk) {
    return row * D + ((chunk ^ k8_swz<D>(row)) << 4);
}
template <int D>
__device__ __forceinline__ int v8_off(int row, int chunk) {
    return row * D + ((chunk ^ v8_swz<D>(row)) << 4);
}

// Key read by lane l32 of a 32-key block.  With this order, register r of
// the score accumulator of a lane in half hi holds key 16 hi + r: each lane
// owns 16 consecutive keys of the block, which is the order the e4m3 P V
// product takes them in (positions 0..15 of its 32-byte B operand).
__device__ __forceinline__ constexpr int key_perm(int m) {
    return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3);
}

// One workgroup = NW waves = 32 NW query rows of one (batch, head); K and V
// tiles of BC keys pass through double-buffered LDS (buffer-to-LDS copies).
// Scores are computed transposed, S^T = K Q^T, so each lane owns one query
// row; the output is accumulated transposed, O^T = V^T P^T.  The query block
// scale is uniform over a wave (its 32 rows lie in one 64-row block), the key
// block scale is uniform over each 64-key half of a tile: both fold into the
// exponent's multiplier.  The value block scales fold into the exponent's
// offset as log2(s_v / s_vmax) <= 0 (and out of the row sum again), and the
// head's largest value scale s_vmax multiplies the output at the end.
template <int D, bool CAUSAL, int NW, int BC, typename TO, int WPE>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(WPE)))
fwd8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K,
            const uint8_t* __restrict__ V, const float* __restrict__ SQ,
            const float* __restrict__ SK, const float* __restrict__ SV,
            uint16_t* __restrict__ O, float* __restrict__ LSE,
            int B, int Hq, int Hkv, int N, float cl2) {
    constexpr int BR = 32 * NW;
    constexpr int CPR = D / 16;
    constexpr int TILE = BC * D;
    constexpr int STAGE = 2 * TILE;
    constexpr int NKB = BC / 32;
    constexpr int NKS = D / 64;
    constexpr int NDB = D / 32;
    constexpr int NH = BC / 64;
    constexpr int WI = TILE / 1024;
    static_assert(WI % NW == 0, "tile copies split evenly over the waves");
    constexpr int IPW = WI / NW;
    static_assert(2 * STAGE <= 65536, "both buffers addressable by immediate offsets");
    static_assert(BR % BC == 0 && BC % 64 == 0, "row blocks start on a key-tile boundary");

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
    const int qb = CAUSAL ? (nqb - 1 - qb_raw) : qb_raw;  // longest rows first
    const int h = bh % Hq;
    const int b = bh / Hq;
    const int hk = h / (Hq / Hkv);

    const size_t qoff = ((size_t)b * Hq + h) * (size_t)N * D;
    const size_t koff = ((size_t)b * Hkv + hk) * (size_t)N * D;
    const uint32_t head_bytes = (uint32_t)N * D;
    const Buf Qb(Q + qoff, head_bytes), Kb(K + koff, head_bytes), Vb(V + koff, head_bytes);

    const int q0 = qb * BR;
    const int qw = q0 + 32 * wave;
    const int q = qw + l32;

    const int nblk = (N + kQBlk - 1) / kQBlk;
    const float* sk_h = SK + (size_t)(b * Hkv + hk) * nblk;
    const float* sv_h = SV + (size_t)(b * Hkv + hk) * nblk;
    const float sq = SQ[(size_t)(b * Hq + h) * nblk + min(qw / kQBlk, nblk - 1)];
    float svmax = 0.f;
    for (int i = lane; i < nblk; i += 64) svmax = fmaxf(svmax, sv_h[i]);
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) svmax = fmaxf(svmax, __shfl_xor(svmax, m, 64));
    const float lsv = __log2f(svmax);

    i32x8 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
        qf[ks] = cat8(Qb.load16((uint32_t)(q * D + 64 * ks + 32 * hi)),
                      Qb.load16((uint32_t)(q * D + 64 * ks + 32 * hi + 16)));

    const int kv_len = CAUSAL ? min(N, q0 + BR) : N;
    const int ntiles = (kv_len + BC - 1) / BC;
    const int nfull = min(CAUSAL ? q0 / BC : ntiles, N / BC);

    uint32_t cpk[IPW], cpv[IPW];
#pragma unroll
    for (int i = 0; i < IPW; ++i) {
        const int p = (wave + NW * i) * 64 + lane;
        const int row = p / CPR, cs = p % CPR;
        cpk[i] = (uint32_t)(row * D + 16 * (cs ^ k8_swz<D>(row)));
        cpv[i] = (uint32_t)(row * D + 16 * (cs ^ v8_swz<D>(row)));
    }
    // Block scales of the tile being copied are loaded with it (vector
    // loads, so that waits on LDS reads stay fine-grained); they become the
    // current tile's when the next copy is issued.
    const Buf SKb(sk_h, (uint32_t)nblk * 4), SVb(sv_h, (uint32_t)nblk * 4);
    float skc[NH], svc[NH], skn[NH], svn[NH];
#pragma unroll
    for (int t = 0; t < NH; ++t) skn[t] = svn[t] = 1.f;
    auto issue = [&](int k0, int buf) {
        unsigned char* base = smem + buf * STAGE;
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            skc[t] = skn[t];
            svc[t] = svn[t];
        }
#pragma unroll
        for (int i = 0; i < IPW; ++i) {
            const int bi = wave + NW * i;
            const uint32_t rowb = (uint32_t)k0 * D;
            buf_to_lds16(Kb, base + bi * 1024, rowb + cpk[i]);
            buf_to_lds16(Vb, base + TILE + bi * 1024, rowb + cpv[i]);
        }
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            const uint32_t blk = (uint32_t)min(k0 / kQBlk + t, nblk - 1);
            skn[t] = SKb.load_f32(blk * 4);
            svn[t] = SVb.load_f32(blk * 4);
        }
    };

    // lane parts of the LDS addresses: K row key_perm(l32) (+ 32 kb, an
    // immediate), chunks 4 ks + 2 hi (+ 1); V rows 16 hi + s / 2 (+ 64 t +
    // 32 (m / 2) + 8 (m % 2), immediates), chunk 2 cb + (lane / 16) % 2,
    // byte 8 (s % 2), with s = lane % 16
    uint32_t ko[NKS][2], vo[NDB];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int e = 0; e < 2; ++e) ko[ks][e] = lds_lane_off((uint32_t)k8_off<D>(key_perm(l32), 4 * ks + 2 * hi + e));
    {
        const int s16 = lane & 15;
        const int g16 = (lane >> 4) & 1;
#pragma unroll
        for (int cb = 0; cb < NDB; ++cb)
            vo[cb] = lds_lane_off((uint32_t)(v8_off<D>(16 * hi + (s16 >> 1), 2 * cb + g16) + 8 * (s16 & 1)));
    }

    f32x16 o[NDB];
#pragma unroll
    for (int cb = 0; cb < NDB; ++cb) o[cb] = zero16();
    float m_s = -INFINITY;
    float l_s = 0.f;
    const float cq = cl2 * sq;

    // Tile j from the buffer at cur.  The tile's LDS reads go through this
    // restrict-qualified pointer, so the compiler does not make the
    // transposing reads wait for the copies of the next tile into the other
    // buffer.
    auto body_at = [&](const unsigned char* __restrict__ cur, int j, auto mask_tag)
                       __attribute__((always_inline)) {
        constexpr bool MASK = decltype(mask_tag)::value;
        const int k0 = j * BC;
        const unsigned char* kbase = cur;
        const unsigned char* vbase = cur + TILE;

        // exponent multiplier and value-scale offset of each 64-key half
        float c[NH], e[NH];
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            c[t] = cq * skc[t];
            e[t] = __log2f(svc[t]) - lsv;
        }

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const u32x4 a0 = *reinterpret_cast<const u32x4*>(kbase + ko[ks][0] + 32 * kb * D);
                const u32x4 a1 = *reinterpret_cast<const u32x4*>(kbase + ko[ks][1] + 32 * kb * D);
                s[kb] = mma8(cat8(a0, a1), qf[ks], s[kb]);
            }
        if (MASK) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + 32 * kb + 16 * hi + r;
                    if ((CAUSAL && key > q) || key >= N) s[kb][r] = -INFINITY;
                }
        }

        // V^T operands, read just before each product
        auto read_v = [&](int t, int cb) {
            i32x8 r;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const i32x2 x = lds_read_tr8(vbase + vo[cb] + (64 * t + 32 * (m >> 1) + 8 * (m & 1)) * D);
                r[2 * m] = x[0];
                r[2 * m + 1] = x[1];
            }
            return r;
        };

        float mx = -INFINITY;
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            float mh = -INFINITY;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int r = 0; r < 16; ++r) mh = fmaxf(mh, s[2 * t + kk][r]);
            mx = fmaxf(mx, mh * c[t]);
        }
        const float mt = halves_max(mx);

        if (__any(mt > m_s + kTau8)) {
            const float mn = fmaxf(m_s, mt);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_s - mn);
            l_s *= alpha;
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
                for (int r = 0; r < 16; ++r) o[cb][r] *= alpha;
            m_s = mn;
        }
        const float mu = (m_s == -INFINITY) ? 0.f : m_s;

        i32x8 pb[NH];
#pragma unroll
        for (int t = 0; t < NH; ++t) {
            const float bias = kPOff + e[t] - mu;
            float ls = 0.f;
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int w = 0; w < 4; ++w) {
                    float p[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) p[i] = fast_exp2(fmaf(s[2 * t + kk][4 * w + i], c[t], bias));
                    ls += (p[0] + p[1]) + (p[2] + p[3]);
                    pb[t][4 * kk + w] = pack4_e4m3(p[0], p[1], p[2], p[3]);
                }
            l_s += ls * fast_exp2(-e[t]);
        }

#pragma unroll
        for (int t = 0; t < NH; ++t)
#pragma unroll
            for (int cb = 0; cb < NDB; ++cb)
                o[cb] = mma8(read_v(t, cb), pb[t], o[cb]);
    };
    // tile j in buffer BUFC, or (BUFC < 0) in buffer j & 1
    auto body = [&](int j, auto mask_tag, auto buf_tag) __attribute__((always_inline)) {
        constexpr int BUFC = decltype(buf_tag)::value;
        body_at(smem + (BUFC >= 0 ? BUFC : (j & 1)) * STAGE, j, mask_tag);
    };

    issue(0, 0);
    wait_vmem();
    __syncthreads();

    // The copy of the next tile is issued at the start of every tile, also
    // the last (the extra tile lies in this head's range or past its end,
    // reads as zeros, and lands in the buffer no later tile reads).
    int j = 0;
    for (; j + 1 < nfull; j += 2) {
        issue((j + 1) * BC, 1);
        body(j, std::false_type{}, std::integral_constant<int, 0>{});
        wait_vmem();
        __syncthreads();
        issue((j + 2) * BC, 0);
        body(j + 1, std::false_type{}, std::integral_constant<int, 1>{});
        wait_vmem();
        __syncthreads();
    }
    for (; j < ntiles; ++j) {
        issue((j + 1) * BC, (j + 1) & 1);
        if (!CAUSAL || j * BC <= qw + 31) body(j, std::true_type{}, std::integral_constant<int, -1>{});
        wait_vmem();
        __syncthreads();
    }

    const float l_tot = l_s + swap_halves(l_s);
    if (q < N) {
        const float inv = svmax / l_tot;
        uint16_t* Orow = O + qoff + (size_t)q * D;
#pragma unroll
        for (int cb = 0; cb < NDB; ++cb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                u32x2 w;
                w[0] = Mma<TO>::pack2(o[cb][4 * g] * inv, o[cb][4 * g + 1] * inv);
                w[1] = Mma<TO>::pack2(o[cb][4 * g + 2] * inv, o[cb][4 * g + 3] * inv);
                *reinterpret_cast<u32x2*>(Orow + 32 * cb + 8 * g + 4 * hi) = w;
            }
        if (hi == 0) LSE[(size_t)(b * Hq + h) * N + q] = (m_s - kPOff + __log2f(l_tot)) * kLn2;
    }
}

template <typename T, int D>
hipError_t quant8_d(const Fp8QuantArgs& a) {
    const int nblk = (a.N + kQBlk - 1) / kQBlk;
    const dim3 grid((unsigned)(nblk * a.B * a.H));
    if (a.signs)
        hipLaunchKernelGGL((quant8_kernel<T, D, true>), grid, dim3(64), 0, a.stream,
                           (const uint16_t*)a.x, a.signs, a.rs, a.codes, a.scales, a.N, nblk);
    else
        hipLaunchKernelGGL((quant8_kernel<T, D, false>), grid, dim3(64), 0, a.stream,
                           (const uint16_t*)a.x, a.signs, a.rs, a.codes, a.scales, a.N, nblk);
    return hipGetLastError();
}

template <int D, bool CAUSAL, int BC, typename TO, int NW, int WPE>
hipError_t fwd8_launch(const Fp8FwdArgs& a) {
    const int nqb = (a.N + 32 * NW - 1) / (32 * NW);
    const int total = nqb * a.Hq * a.B;
    hipLaunchKernelGGL((fwd8_kernel<D, CAUSAL, NW, BC, TO, WPE>), dim3((unsigned)total), dim3(NW * 64), 0,
                       a.stream, a.q, a.k, a.v, a.sq, a.sk, a.sv, (uint16_t*)a.o, a.lse, a.B, a.Hq,
                       a.Hkv, a.N, a.cl2);
    return hipGetLastError();
}

template <int D, typename TO>
hipError_t fwd8_d(const Fp8FwdArgs& a) {
    // key tile: 64 keys at D = 128, 128 keys at D = 64 (8 KB per K or V tile).
    // 4-wave workgroups at 3 waves per SIMD, V^T read just before each P V
    // product (the softmax of one wave hides under the products of the other
    // two).
    constexpr int BC = D == 64 ? 128 : 64;
    return a.causal ? fwd8_launch<D, true, BC, TO, 4, 3>(a) : fwd8_launch<D, false, BC, TO, 4, 3>(a);
}

}  // namespace

hipError_t launch_fp8_quantize(const Fp8QuantArgs& a) {
    const bool bf = a.dtype == 2;
    if (a.d == 128) return bf ? quant8_d<BF16, 128>(a) : quant8_d<FP16, 128>(a);
    return bf ? quant8_d<BF16, 64>(a) : quant8_d<FP16, 64>(a);
}

hipError_t launch_fwd_fp8(const Fp8FwdArgs& a) {
    const bool bf = a.out_dtype == 2;
    if (a.d == 128) return bf ? fwd8_d<128, BF16>(a) : fwd8_d<128, FP16>(a);
    return bf ? fwd8_d<64, BF16>(a) : fwd8_d<64, FP16>(a);
}

}  // namespace fa355
