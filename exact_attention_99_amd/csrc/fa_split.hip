// Split-KV forward (FlashDecoding): for few query rows and a long key/value
// sequence, the key range is cut into chunks that are processed in parallel,
// each producing a partial output normalised over its own keys plus the
// logsumexp of its scores; a second pass merges the partials with the same
// rescale the online softmax uses ("FlashAttention" glossary, the
// FlashDecoding paragraph; "FlashAttention 1, 2, and 3 Explained", section 2,
// the online-softmax update).
//
// Rows: the G query heads that share a K/V head are stacked into the rows of
// one tile (row r = g * N_q + i for query head hk * G + g and query i), which
// is possible because those heads' rows are contiguous in [B, H_q, N_q, d].
// Causal alignment for N_q <= N_kv: query i is the (N_kv - N_q + i)-th
// position of the sequence, so it sees keys j <= i + N_kv - N_q.
#include "fa_common.h"
#include "fa_launch.h"

namespace fa355 {
namespace {

// One wave per workgroup: partial attention of 32 stacked rows over the keys
// [c0, c1) of one chunk.  K and V tiles of BC keys stream through a ring of NS
// LDS stages by buffer-to-LDS copies (keys past N_kv read as zeros and are
// masked, as are keys of the next chunk): tile j waits for its own copies,
// then issues those of tile j + NS - 1 and is computed while they fly.  Two
// stages measure best; three or four (more bytes in flight, fewer workgroups
// per compute unit) are slower.
template <typename T, int D, bool CAUSAL>
__global__ void __launch_bounds__(64)
fwd_split16_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                   const uint16_t* __restrict__ V, float* __restrict__ Opart,
                   float* __restrict__ Lpart, int B, int Hq, int Hkv, int Nq, int Nkv, int chunk,
                   int nrb, float cl2) {
    constexpr int BC = 4096 / D;              // 8 KB per K or V tile
    constexpr int KCH = D / 8;
    constexpr int TILE = BC * D * 2;
    constexpr int STAGE = 2 * TILE;
    constexpr int NKB = BC / 32;
    constexpr int NKG = BC / 16;
    constexpr int NDB = D / 32;
    constexpr int NKS = D / 16;
    constexpr int WI = TILE / 1024;           // 1 KB wave copies per tile
    constexpr int NS = FA355_SPLIT_NS;        // LDS stages
    constexpr int CPT = 2 * WI;               // copies per tile (K and V)
    static_assert(NS >= 2 && (NS - 1) * CPT <= 63, "copies in flight fit the vector-memory counter");

    __shared__ __attribute__((aligned(16))) unsigned char smem[NS * STAGE];

    const int lane = threadIdx.x;
    const int l32 = lane & 31;
    const int hi = lane >> 5;

    const int split = blockIdx.x / nrb;
    const int rb = blockIdx.x % nrb;
    const int hk = blockIdx.y % Hkv;
    const int b = blockIdx.y / Hkv;
    const int G = Hq / Hkv;
    const int rows = G * Nq;
    const int r = 32 * rb + l32;              // this lane's stacked row
    const int qi = r % Nq;                    // its query index
    const size_t row0 = ((size_t)b * Hq + (size_t)hk * G) * Nq;   // first row of the group
    const size_t nrows_all = (size_t)B * Hq * Nq;

    const Buf Qb(Q + row0 * D, (uint32_t)rows * D * 2);
    u32x4 qf[NKS];
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) qf[ks] = Qb.load16((uint32_t)(r * D + 16 * ks + 8 * hi) * 2);

    const size_t kvoff = ((size_t)b * Hkv + hk) * (size_t)Nkv * D;
    const uint32_t head_bytes = (uint32_t)Nkv * D * 2;
    const Buf Kb(K + kvoff, head_bytes), Vb(V + kvoff, head_bytes);

    const int c0 = split * chunk;
    const int c1 = min(Nkv, c0 + chunk);
    const int ntiles = c1 > c0 ? (c1 - c0 + BC - 1) / BC : 0;
    const int shift = Nkv - Nq;               // causal: key j visible iff j <= qi + shift

    auto issue = [&](int k0, int buf) {
        unsigned char* base = smem + buf * STAGE;
#pragma unroll
        for (int i = 0; i < WI; ++i) {
            const int p = i * 64 + lane;
            const int row = p / KCH, pc = p % KCH;
            const uint32_t rowb = (uint32_t)(k0 + row) * D * 2;
            buf_to_lds16(Kb, base + i * 1024, rowb + (kq_off<D>(row, pc) - row * D * 2));
            buf_to_lds16(Vb, base + TILE + i * 1024, rowb + 16 * (pc ^ tr_swz<D>(row)));
        }
    };

    const int g16 = lane >> 4;
    const int j16 = lane & 15;
    const int tr_row = 4 * hi + (j16 >> 2);
    const int tr_col = 2 * (16 * (g16 & 1) + 4 * (j16 & 3));

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = zero16();
    float m_s = -INFINITY;
    float l_s = 0.f;

#pragma unroll
    for (int j = 0; j < NS - 1; ++j)
        if (j < ntiles) issue(c0 + j * BC, j);
    // One tile from the buffer at cur.  Its LDS reads go through this
    // restrict-qualified pointer, so the compiler does not make the transposing
    // reads wait for the copy of the next tile into the other buffer.
    auto tile = [&](const unsigned char* __restrict__ cur, int k0) __attribute__((always_inline)) {
        const unsigned char* ks_base = cur;
        const unsigned char* vt_base = cur + TILE;

        f32x16 s[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                const u32x4 a = *reinterpret_cast<const u32x4*>(ks_base + kq_off<D>(32 * kb + l32, 2 * ks + hi));
                s[kb] = Mma<T>::mma(a, qf[ks], s[kb]);
            }
        // keys past the chunk (or the sequence), and under the causal mask
        // keys after this row's position
        const bool need_mask = (k0 + BC > c1) || (CAUSAL && k0 + BC - 1 > shift);
        if (need_mask) {
            asm volatile("" ::: "memory");
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) {
                    const int key = k0 + 32 * kb + acc_row(rr, hi);
                    if (key >= c1 || (CAUSAL && key > qi + shift)) s[kb][rr] = -INFINITY;
                }
        }

        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[kb][rr]);
        const float mt = halves_max(mx) * cl2;
        if (__any(mt > m_s + kTau)) {
            const float mn = fmaxf(m_s, mt);
            const float alpha = (mn == -INFINITY) ? 1.f : fast_exp2(m_s - mn);
            l_s *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int rr = 0; rr < 16; ++rr) o[db][rr] *= alpha;
            m_s = mn;
        }
        const float mu = (m_s == -INFINITY) ? 0.f : m_s;

        u32x4 pb[NKG];
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float p0 = fast_exp2(fmaf(s[kb][8 * t + 2 * jj], cl2, -mu));
                    const float p1 = fast_exp2(fmaf(s[kb][8 * t + 2 * jj + 1], cl2, -mu));
                    ls += p0 + p1;
                    pb[2 * kb + t][jj] = Mma<T>::pack2(p0, p1);
                }
        l_s += ls;

#pragma unroll
        for (int kg = 0; kg < NKG; ++kg)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const int row = 16 * kg + tr_row;
                const int col = 64 * db + tr_col;
                const u32x2 lo = lds_read_tr16(vt_base + vt_off<D>(row, col));
                const u32x2 up = lds_read_tr16(vt_base + vt_off<D>(row + 8, col));
                u32x4 a;
                a[0] = lo[0]; a[1] = lo[1]; a[2] = up[0]; a[3] = up[1];
                o[db] = Mma<T>::mma(a, pb[kg], o[db]);
            }
    };
    // tile j waits only for its own copies: the copies of the tiles after it
    // (at most NS - 2 of them issued yet, in issue order) may stay in flight
    for (int j = 0; j < ntiles; ++j) {
        const int k0 = c0 + j * BC;
        const int later = min(NS - 2, ntiles - 1 - j);
        static_for<NS - 1>([&](auto lc) {
            constexpr int L = decltype(lc)::value;
            if (later == L) wait_vmem_n<L * CPT>();
        });
        __syncthreads();
        if (j + NS - 1 < ntiles) issue(k0 + (NS - 1) * BC, (j + NS - 1) % NS);
        tile(smem + (j % NS) * STAGE, k0);
    }

    // partial result of this chunk: O normalised over the chunk's keys and
    // the natural-log logsumexp of its scores (-inf and 0 if it saw none)
    const float l_tot = l_s + swap_halves(l_s);
    if (r < rows) {
        const bool any = l_tot > 0.f;
        const float inv = any ? 1.f / l_tot : 0.f;
        const size_t R = row0 + r;
        float* orow = Opart + ((size_t)split * nrows_all + R) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                f32x4 w;
#pragma unroll
                for (int i = 0; i < 4; ++i) w[i] = o[db][4 * g + i] * inv;
                *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * g + 4 * hi) = w;
            }
        if (hi == 0)
            Lpart[(size_t)split * nrows_all + R] = any ? (m_s + __log2f(l_tot)) * kLn2 : -INFINITY;
    }
}

// Merge of the partials of one row per 256-thread workgroup:
// lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s, rounded to the
// output dtype.  The work is a few dependent memory round trips, so every
// load is issued before anything waits on one: thread t takes output
// dimensions 4 (t % TPD) .. + 3 of the chunks g, g + NG, g + 2 NG, ...
// (g = t / TPD) as 16-byte loads, up to MB chunks at a time, while wave 0
// reads the chunks' logsumexps (chunk s in lane s % 64) and forms the weights
// exp(lse_s - max) into LDS.  Each thread sums its chunks, then the NG group
// sums are added in LDS in group order.
constexpr int kMaxSplits = 1024;

template <typename T, int D>
__global__ void __launch_bounds__(256)
merge_split_kernel(const float* __restrict__ Opart, const float* __restrict__ Lpart,
                   uint16_t* __restrict__ O, float* __restrict__ LSE, int nrows, int nsplit) {
    constexpr int TPD = D / 4;         // threads per partial row
    constexpr int NG = 256 / TPD;      // chunk groups
    constexpr int MB = 8;              // chunks per thread per batch
    constexpr int LPL = kMaxSplits / 64;
    __shared__ float w[kMaxSplits];
    __shared__ float red[2];
    __shared__ f32x4 part[NG][TPD];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int R = blockIdx.x;
    const int g = tid / TPD, c4 = tid % TPD;
    const float* ob = Opart + (size_t)R * D + 4 * c4;
    const size_t cstride = (size_t)nrows * D;   // floats between chunks

    auto load_batch = [&](int s0, f32x4 (&buf)[MB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int s = s0 + g + NG * i;
            buf[i] = s < nsplit ? *reinterpret_cast<const f32x4*>(ob + (size_t)s * cstride) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
    };
    f32x4 pb[MB];
    load_batch(0, pb);

    if (tid < 64) {
        float lv[LPL];
#pragma unroll
        for (int k = 0; k < LPL; ++k) {
            const int s = lane + 64 * k;
            lv[k] = (64 * k < nsplit && s < nsplit) ? Lpart[(size_t)s * nrows + R] : -INFINITY;
        }
        float m = -INFINITY;
#pragma unroll
        for (int k = 0; k < LPL; ++k) m = fmaxf(m, lv[k]);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o, 64));
        float ws = 0.f;
#pragma unroll
        for (int k = 0; k < LPL; ++k) {
            const int s = lane + 64 * k;
            if (64 * k < nsplit && s < nsplit) {
                const float x = (lv[k] == -INFINITY || m == -INFINITY) ? 0.f : __expf(lv[k] - m);
                w[s] = x;
                ws += x;
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) ws += __shfl_xor(ws, o, 64);
        if (lane == 0) {
            red[0] = m;
            red[1] = ws;
        }
    }
    __syncthreads();

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0;; s0 += NG * MB) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const int s = s0 + g + NG * i;
            if (s < nsplit) {
                const float ws = w[s];
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[e] = fmaf(ws, pb[i][e], acc[e]);
            }
        }
        if (s0 + NG * MB >= nsplit) break;
        load_batch(s0 + NG * MB, pb);
    }
    part[g][c4] = acc;
    __syncthreads();
    if (g == 0) {
        f32x4 t = part[0][c4];
#pragma unroll
        for (int gg = 1; gg < NG; ++gg)
#pragma unroll
            for (int e = 0; e < 4; ++e) t[e] += part[gg][c4][e];
        const float wsum = red[1];
        const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
        u32x2 out;
        out[0] = Mma<T>::pack2(t[0] * inv, t[1] * inv);
        out[1] = Mma<T>::pack2(t[2] * inv, t[3] * inv);
        *reinterpret_cast<u32x2*>(O + (size_t)R * D + 4 * c4) = out;
        if (c4 == 0) LSE[R] = wsum > 0.f ? red[0] + __logf(wsum) : -INFINITY;
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t split16(const SplitArgs& a) {
    constexpr int BC = 4096 / D;
    const int G = a.Hq / a.Hkv;
    const int nrb = (G * a.Nq + 31) / 32;
    hipLaunchKernelGGL((fwd_split16_kernel<T, D, CAUSAL>), dim3((unsigned)(a.nsplit * nrb), (unsigned)(a.B * a.Hkv)),
                       dim3(64), 0, a.stream, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                       a.opart, a.lpart, a.B, a.Hq, a.Hkv, a.Nq, a.Nkv, a.chunk, nrb, a.cl2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    (void)BC;
    const int nrows = a.B * a.Hq * a.Nq;
    hipLaunchKernelGGL((merge_split_kernel<T, D>), dim3((unsigned)nrows), dim3(256), 0, a.stream,
                       a.opart, a.lpart, (uint16_t*)a.o, a.lse, nrows, a.nsplit);
    return hipGetLastError();
}

template <typename T>
hipError_t split16d(const SplitArgs& a) {
    if (a.d == 64) return a.causal ? split16<T, 64, true>(a) : split16<T, 64, false>(a);
    return a.causal ? split16<T, 128, true>(a) : split16<T, 128, false>(a);
}

}  // namespace

int split_tile_keys(int d) { return 4096 / d; }

hipError_t launch_fwd_split(const SplitArgs& a) {
    return a.dtype == 2 ? split16d<BF16>(a) : split16d<FP16>(a);
}

}  // namespace fa355
