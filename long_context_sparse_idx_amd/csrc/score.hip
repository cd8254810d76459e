// Indexer score kernels for gfx950.
//
//   S[b,t,s] = sum_h w[b,t,h] * max(0, q[b,t,h,:] . k[b,s,:])   for s <= p_t
//
// (The pages name the indexer only as a dot product followed by a top-k --
// IndexShare term page (earlyterms.com), opening definition -- and place it
// in front of every layer's attention, scanning the whole context --
// IndexCache news article (app.myzaker.com), section "IndexCache".)
//
// The contraction over d is dense, so it runs on bf16 MFMA
// (v_mfma_f32_32x32x16_bf16).  A wave owns 64 "rows" = (query, head) pairs
// with heads contiguous (64/H queries per wave) as the MFMA M dimension, keys
// are the N dimension (32 per block), d is K.  The ReLU, the per-head weight
// and the head reduction run in the epilogue on the fp32 accumulators, so
// per-head scores never leave registers; only the head-reduced row is
// written (fp32, one row of ld floats per query).
//
// fp8 keys: every OCP E4M3 value is exactly a bf16 value, so keys are widened
// to bf16 on load and the per-key scale is applied after the head reduction
// (max(0, a x) = a max(0, x) for a > 0).
//
// fp8 keys and fp8 queries: the products run on v_mfma_f32_32x32x64_f8f6f4
// (format 0 = E4M3 on both operands, no block scales) at twice the bf16
// rate; each (token, head) scale is folded into that head's weight and the
// key scale is applied after the head reduction, as above.  For that
// instruction a lane holds 32 bytes of row/column (lane % 32), k-slots of
// group g; the d index behind slot e of step s is g*D/2 + 32*s + e, again
// the same on both operands.
//
// Lane layouts (32x32x16 bf16 MFMA, wave64, g = lane / 32):
//   A (Q):  lane holds row (lane % 32), 8 consecutive k-slots of group g
//   B (K):  lane holds column (lane % 32), the same 8 k-slots of group g
//   D:      lane holds column (lane % 32), rows 8*(r/4) + 4*g + (r%4), r < 16
// Both operands use the same map from (group g, k-step s, k-slot e) to the d
// index, so the MFMA still sums all D products:
//   bf16 keys:  d = 16*s + 8*g + e  -- the two lanes of one key read adjacent
//               16-byte chunks, so one load instruction of a wave touches 32
//               bytes of each of its 32 keys (the split-key kernel reads its
//               keys straight from memory this way: half the distinct cache
//               lines per instruction of the split-halves map, 9 % less time
//               at 131K keys);
//   fp8 keys (widened to bf16): d = g*D/2 + 8*s + e -- each lane reads one
//               contiguous half of the key row (64 B for D = 128).
// Every kernel of one key format uses the same map, so their scores are
// bit-identical.
#include <type_traits>

#include "device_common.h"
#include "kernels.h"

namespace lcsi {

namespace {

constexpr int WAVES_PREFILL = 8;  // 512 threads: 2 waves per SIMD
constexpr int WAVES_SPLIT = 4;
// Split-key kernel: register buffers per wave (the blocks in flight plus the
// one computing) and the waves per SIMD the register allocation must allow
// (1: no limit), per key format.  At 131K bf16 / 1M fp8 keys with 64 heads,
// three buffers at two waves per SIMD were best; four to eight buffers at
// one wave per SIMD lost 3-17 %, and fp8 keys without the two-wave bound
// (more registers, one wave) lost 9 %.
constexpr int SPLIT_NB_BF16 = 3, SPLIT_OCC_BF16 = 1;
constexpr int SPLIT_NB_F8 = 3, SPLIT_OCC_F8 = 2;
// workgroups a split-key call aims for: two per CU in one round (with 256,
// one per CU, 1M fp8 keys took 30 % longer)
constexpr int SPLIT_WGS = 512;

// Operand formats: bf16 keys and queries; fp8 keys widened to bf16; fp8
// keys and fp8 queries on fp8 MFMA.
enum Fmt { F_BF16 = 0, F_K8 = 1, F_QK8 = 2 };

template <int D>
struct KeyGeom {
    static constexpr int KSTEPS = D / 16;     // bf16 MFMA k-steps
    static constexpr int KSTEPS8 = D / 64;    // fp8 MFMA k-steps
    static constexpr int HALF = D / 2;        // d-elements per lane group
    static constexpr int ROWB = D * 2 + 16;   // LDS bytes per bf16 key row (+16 B pad)
    static constexpr int ROWB8 = D + 16;      // LDS bytes per fp8 key row (+16 B pad)
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

// Q fragments and per-row weights of one wave (64 rows = 64/H queries); ILV:
// the interleaved d map of bf16 keys (else the split-halves map).
template <int H, int D, bool ILV>
struct WaveRows {
    bf16x8 qa[2][KeyGeom<D>::KSTEPS];
    float wl[2][16];

    __device__ __forceinline__ void load(const ScoreArgs &a, int b, int tq0, int lane)
    {
        const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row = rt * 32 + l32;
            const int t = tq0 + row / H, h = row % H;
            if (t < a.T_q) {
                const uint8_t *base = a.q + b * a.q_sb + (int64_t)t * a.q_st + h * a.q_sh + g * (ILV ? 16 : KeyGeom<D>::HALF * 2);
#pragma unroll
                for (int s = 0; s < KeyGeom<D>::KSTEPS; ++s) qa[rt][s] = as_bf16x8(ld16(base + (ILV ? 32 : 16) * s));
            } else {
#pragma unroll
                for (int s = 0; s < KeyGeom<D>::KSTEPS; ++s) qa[rt][s] = as_bf16x8(u32x4{0, 0, 0, 0});
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = rt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const int tr = tq0 + rr / H, hr = rr % H;
                wl[rt][r] = tr < a.T_q ? a.w[b * a.w_sb + (int64_t)tr * a.w_st + hr] : 0.f;
            }
        }
    }
};

// fp8 variant: Q fragments are 32 bytes per k-step; each head's query scale
// is folded into its weight.
template <int H, int D>
struct WaveRows8 {
    i32x8 qa[2][KeyGeom<D>::KSTEPS8];
    float wl[2][16];

    __device__ __forceinline__ void load(const ScoreArgs &a, int b, int tq0, int lane)
    {
        const int g = lane >> 5, l32 = lane & 31;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
            const int row = rt * 32 + l32;
            const int t = tq0 + row / H, h = row % H;
#pragma unroll
            for (int s = 0; s < KeyGeom<D>::KSTEPS8; ++s) {
                u32x4 lo{0, 0, 0, 0}, hi{0, 0, 0, 0};
                if (t < a.T_q) {
                    const uint8_t *base = a.q + b * a.q_sb + (int64_t)t * a.q_st + h * a.q_sh + g * KeyGeom<D>::HALF + 32 * s;
                    lo = ld16(base);
                    hi = ld16(base + 16);
                }
                qa[rt][s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rr = rt * 32 + 8 * (r >> 2) + 4 * g + (r & 3);
                const int tr = tq0 + rr / H, hr = rr % H;
                wl[rt][r] = tr < a.T_q ? a.w[b * a.w_sb + (int64_t)tr * a.w_st + hr] *
                                             a.q_scale[b * a.qs_sb + (int64_t)tr * a.qs_st + hr]
                                       : 0.f;
            }
        }
    }
};

__device__ __forceinline__ i32x8 lds_ld32(const uint8_t *p)
{
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(p), hi = *reinterpret_cast<const u32x4 *>(p + 16);
    return i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
}

// Epilogue of one 32-key block: ReLU * weight and the head reduction
// (epi_reduce, pure register arithmetic), then the store (epi_store).  The
// summation order is fixed (row tile, then r ascending, then the lane-pair
// add), so every kernel that calls these produces bit-identical scores.
template <int H>
struct Part {
    static constexpr int N = H >= 8 ? 64 / H : 8;
    float v[N];
};

// The epilogue in 32 units, one per accumulator value r of this lane
// (acc0[r] for r < 16, else acc1[r - 16]): unit r adds w * max(0, x) to its
// partial sum.  Units run in ascending r (the prefill kernel spreads them
// over the MFMAs of the next block), then finish() adds the partials.
template <int H>
struct EpiAcc {
    static constexpr int QPW = H >= 8 ? 64 / H : 1;
    static constexpr int E = 32 / QPW;                                       // units per query (H >= 8)
    // partial sums per query: two chains, fed alternately, are enough -- the
    // prefill kernel's units are spread over the next block's MFMAs, so a
    // chain's previous fma has long finished -- and each partial fewer saves
    // an add per block (8 partials: 1.3 % slower at 200K keys, 4: 0.9 %)
    static constexpr int NP = H >= 8 ? 2 : 1;
    static constexpr int NQ = H >= 8 ? QPW : 8;                              // queries of this lane
    float ps[NQ][NP];

    __device__ __forceinline__ void init()
    {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int j = 0; j < NP; ++j) ps[q][j] = 0.f;
    }

    __device__ __forceinline__ void unit(int r, const f32x16 &acc0, const f32x16 &acc1, const float (&wl)[2][16])
    {
        const float m = fmaxf(r < 16 ? acc0[r] : acc1[r - 16], 0.f);
        const float wv = wl[r >> 4][r & 15];
        if constexpr (H >= 8) {
            // Each query owns E accumulator values of this lane, summed into
            // NP independent partial sums (element e goes to partial e % NP).
            const int row = 32 * (r >> 4) + 8 * ((r & 15) >> 2);  // first row of r's group of 4
            const int q = row / H;
            const int e = r - q * E;                               // element index within query q
            ps[q][e % NP] = __builtin_fmaf(wv, m, ps[q][e % NP]);
        } else {
            static_assert(H == 4, "H must be 4, 8, 16, 32 or 64");
            // rows 8j + 4g + i of tile rt are the 4 heads of query 8*rt + 2j + g
            const int rt = r >> 4, j = (r & 15) >> 2;
            ps[rt * 4 + j][0] = __builtin_fmaf(wv, m, ps[rt * 4 + j][0]);
        }
    }

    // the partials added as a balanced tree, the lane halves summed (H >= 8),
    // the key scale applied
    __device__ __forceinline__ Part<H> finish(float kscale)
    {
        Part<H> p;
        if constexpr (H >= 8) {
#pragma unroll
            for (int q = 0; q < QPW; ++q) {
#pragma unroll
                for (int w = NP / 2; w >= 1; w >>= 1)
#pragma unroll
                    for (int j = 0; j < w; ++j) ps[q][j] += ps[q][j + w];
                p.v[q] = sum_lane_halves(ps[q][0]) * kscale;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) p.v[i] = ps[i][0] * kscale;
        }
        return p;
    }
};

template <int H>
__device__ __forceinline__ Part<H> epi_reduce(const f32x16 &acc0, const f32x16 &acc1, const float (&wl)[2][16],
                                              float kscale)
{
    EpiAcc<H> e;
    e.init();
#pragma unroll
    for (int r = 0; r < 32; ++r) e.unit(r, acc0, acc1, wl);
    return e.finish(kscale);
}

// Rows of the score matrix a workgroup writes: rows t_lo .. t_lo + n - 1
// starting at `base`, row stride ld floats.  Stores past them (query rows
// beyond T_q) and masked lanes are dropped by the buffer range check.
struct RowSpan {
    float *base;
    uint32_t bytes;
    int64_t ld;
    int t_lo;
};

template <int H>
__device__ __forceinline__ void epi_store(const Part<H> &p, const RowSpan &rs, bool key_ok, int tq0, int key, int lane)
{
    const int g = lane >> 5;
    auto put = [&](bool mine, int t, float v) {
        const uint32_t off = mine ? (uint32_t)(((int64_t)(t - rs.t_lo) * rs.ld + key) * 4) : rs.bytes;
        store_b32_ranged(rs.base, rs.bytes, off, v);
    };
    if constexpr (H >= 8) {
        constexpr int QPW = 64 / H;
        if constexpr (QPW == 1) {
            put(key_ok && g == 0, tq0, p.v[0]);
        } else {
#pragma unroll
            for (int q = 0; q < QPW; ++q) put(key_ok && (q < QPW / 2) == (g == 0), tq0 + q, p.v[q]);
        }
    } else {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int j = 0; j < 4; ++j) put(key_ok, tq0 + rt * 8 + 2 * j + g, p.v[rt * 4 + j]);
    }
}

template <int D>
__device__ __forceinline__ void mfma_block(const bf16x8 (&qa)[2][KeyGeom<D>::KSTEPS], const bf16x8 (&bk)[KeyGeom<D>::KSTEPS],
                                           f32x16 &acc0, f32x16 &acc1)
{
    acc0 = f32x16{0};
    acc1 = f32x16{0};
#pragma unroll
    for (int s = 0; s < KeyGeom<D>::KSTEPS; ++s) {
        acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bk[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bk[s], acc1, 0, 0, 0);
    }
}

template <int D>
__device__ __forceinline__ void mfma_block8(const i32x8 (&qa)[2][KeyGeom<D>::KSTEPS8], const i32x8 (&bk)[KeyGeom<D>::KSTEPS8],
                                            f32x16 &acc0, f32x16 &acc1)
{
    acc0 = f32x16{0};
    acc1 = f32x16{0};
#pragma unroll
    for (int s = 0; s < KeyGeom<D>::KSTEPS8; ++s) {
        acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[0][s], bk[s], acc0, 0, 0, 0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa[1][s], bk[s], acc1, 0, 0, 0, 0, 0, 0);
    }
}

// ---------------------------------------------------------------------------
// Prefill: one workgroup = 8 waves = 8*64/H consecutive query rows of one
// sequence, sweeping keys 0 .. p_max in tiles staged in a double-buffered LDS
// ring while the next tile is in flight.  Workgroups are issued heaviest
// (last rows) first.  All concurrently running workgroups sweep the keys in
// the same order, so each XCD's L2 serves a key tile to all its workgroups.
//   bf16 keys, and fp8 keys with fp8 queries: 128-key tiles copied straight
//              from memory into LDS (buffer loads to LDS, no staging
//              registers), rows padded by one 16-byte slot so the B-fragment
//              reads are free of bank conflicts (fp8: the tile's key scales
//              follow the rows); the two buffers are separate LDS arrays
//              named at compile time (the tile loop is unrolled by two), so
//              reads of one never wait for the loads filling the other.
//   fp8 keys with bf16 queries: 64-key tiles fetched into registers,
//              widened to bf16 and written to LDS.
// Inside each wave the MFMAs of a 32-key block overlap the epilogue of the
// previous block (software pipeline; the accumulators of block j-1 wait in
// pa0/pa1 while block j runs).
//
// Fused selection (FUSE, H >= 16): instead of the score row, the kernel
// writes each row's candidates for the top-k.
//   1. Sample: when the workgroup's longest row has more than FUSE_CAP keys,
//      it first scores ns whole tiles spread evenly over the keys that all
//      its rows cover into LDS (ns: enough for about 24 sampled scores above
//      a row's k-th largest, between 4 and NS = SPQ / KT), and each wave takes,
//      for each of its query rows, the r-th largest sampled score as the
//      row's threshold tau.  r is the expected number of sampled scores at
//      or above the row's k-th largest, plus 4.5 standard deviations and 2,
//      so that the top-k lies at or above tau with high probability while
//      the number of scores at or above tau stays far below FUSE_CAP.  Rows
//      of shorter workgroups keep every score (tau = -inf).
//   2. Sweep: the full causal sweep, whose epilogue writes every score >= tau
//      of a key at or before the row's position as a (score bits, position)
//      pair to the row's candidate slots, in ascending position order (one
//      ballot and prefix count per 32-key block), and at the end the count.
// Every score that reaches the row's k-th largest is a candidate whenever
// the count is at least k, so the top-k of the candidates is the top-k of
// the row.  A count below k or above FUSE_CAP only costs time: the caller
// rescores those rows in full (fused_row_bad).
// ---------------------------------------------------------------------------
constexpr int FUSE_SAMPLES = 32768;  // sampled scores per workgroup, 16 bits each (64 KB of LDS)

// Sampled scores are kept as their upper 16 bits (a float truncated toward
// zero: monotone, so order statistics of the truncated values bound those
// of the scores closely; the threshold only steers the candidate count, the
// count decides whether the candidates are used).  ok16: the 16-bit
// order-preserving key of such a value (-0 folded onto +0).
__device__ __forceinline__ uint32_t ok16(uint32_t h)
{
    if (h == 0x8000u) h = 0u;
    return (h & 0x8000u) ? (~h & 0xFFFFu) : (h | 0x8000u);
}

template <int SPQ>
__device__ __forceinline__ float sample_threshold(const uint16_t *s, int ns, int r, int lane)
{
    // the r-th largest of the ns (<= SPQ) sampled keys, bit by bit from the
    // top: the largest key T that at least r samples reach (unused slots
    // count as key 0, below every candidate T)
    uint32_t kk[SPQ / 64];
#pragma unroll
    for (int j = 0; j < SPQ / 64; ++j) kk[j] = 64 * j + lane < ns ? ok16(s[64 * j + lane]) : 0u;
    uint32_t T = 0;
#pragma unroll 1
    for (int bit = 15; bit >= 0; --bit) {
        const uint32_t c = T | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int j = 0; j < SPQ / 64; ++j) cnt += __popcll(ballot(kk[j] >= c));
        if (cnt >= r) T = c;
    }
    const uint32_t h = (T & 0x8000u) ? (T & 0x7FFFu) : (~T & 0xFFFFu);
    return __uint_as_float(h << 16);
}

template <int H, int D, int F, bool FUSE>
__global__ __launch_bounds__(WAVES_PREFILL * 64) void score_prefill_kernel(ScoreArgs a)
{
    using G = KeyGeom<D>;
    constexpr bool Q8 = F == F_QK8;
    constexpr bool DMA = F != F_K8;
    constexpr bool ILV = F == F_BF16;                  // interleaved d map
    constexpr int QPW = 64 / H;
    constexpr int QPB = WAVES_PREFILL * QPW;
    constexpr int NT = WAVES_PREFILL * 64;
    constexpr int KT = (!DMA || H < 16) ? 64 : 128;   // keys per LDS tile
    constexpr int ROWB = Q8 ? G::ROWB8 : G::ROWB;     // LDS bytes per key row
    constexpr int SCB = Q8 ? KT * 4 : 0;               // key scales after the rows (fp8 x fp8)
    constexpr int SPB = H >= 8 ? QPW : 8;              // score stores per 32-key block and wave
    constexpr int SPQ = FUSE ? FUSE_SAMPLES / QPB : 64;  // sampled keys per query row
    constexpr int NS = SPQ / KT;                       // sampled tiles
    static_assert(!FUSE || (H >= 16 && SPQ % KT == 0 && SPQ % 64 == 0), "fused sample shape");

    __shared__ __attribute__((aligned(1024))) uint8_t sk0[KT * ROWB + SCB];
    __shared__ __attribute__((aligned(1024))) uint8_t sk1[KT * ROWB + SCB];
    __shared__ float ssc[2][F == F_K8 ? KT : 1];
    __shared__ uint16_t samp[FUSE ? FUSE_SAMPLES : 1];

    // (the wave index as a scalar: addresses built from it, such as a
    // buffer resource, are then known to be the same in every lane)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, l32 = lane & 31,
              g = lane >> 5;
    const int b = blockIdx.y;
    const int t0 = (gridDim.x - 1 - blockIdx.x) * QPB;
    const int t_end = min(a.T_q, t0 + QPB);
    const int64_t n_keys = a.q_pos0 + t_end;
    const int ntiles = (int)((n_keys + KT - 1) / KT);
    const uint8_t *kb = a.k + b * a.k_sb;

    if constexpr (!FUSE) {
        // rescoring after a fused pass, when its list of unsettled rows
        // overflowed: only workgroups holding such a row
        if (a.redo) {
            if (*a.rcount <= a.rmax) return;
            bool any = false;
            for (int t = t0; t < t_end; ++t)
                any |= fused_row_bad(a.redo[(int64_t)b * a.T_q + t], a.q_pos0 + t + 1, a.top_k);
            if (!any) return;
        }
    }

    typename std::conditional<Q8, WaveRows8<H, D>, WaveRows<H, D, ILV>>::type rows;
    const int tq0 = t0 + wave * QPW;
    rows.load(a, b, tq0, lane);

    float *Sb = a.S + (int64_t)b * a.T_q * a.ld;
    const RowSpan rs{Sb + (int64_t)t0 * a.ld, (uint32_t)((t_end - t0) * a.ld * 4), a.ld, t0};
    f32x16 pa0 = f32x16{0}, pa1 = f32x16{0};
    int pkey = -1;
    float pks = 1.f;

    // One 32-key block of the tile at `tb`: B fragments from LDS, the MFMAs,
    // interleaved with the epilogue (ReLU * w, head reduction) of the
    // previous block, whose reduced scores go to `sink` with that block's
    // key (-1 before the first block).  The interleave is fixed in the code:
    // each MFMA is followed by its share of the epilogue units and a
    // scheduling barrier, so the VALU work of one wave fills the MFMA
    // pipeline's shadow whatever the surrounding control flow.
    auto block = [&](const uint8_t *tb, int cb, float ksc, int key, auto &sink) {
        const uint8_t *src = tb + (cb * 32 + l32) * ROWB + g * (Q8 ? G::HALF : (ILV ? 16 : G::HALF * 2));
        f32x16 acc0 = f32x16{0}, acc1 = f32x16{0};
        EpiAcc<H> ea;
        ea.init();
        if constexpr (Q8) {
            constexpr int NMF = 2 * G::KSTEPS8, UPM = 32 / NMF;
            i32x8 bk[G::KSTEPS8];
#pragma unroll
            for (int s = 0; s < G::KSTEPS8; ++s) bk[s] = lds_ld32(src + 32 * s);
#pragma unroll
            for (int i = 0; i < NMF; ++i) {
                if (i % 2 == 0)
                    acc0 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(rows.qa[0][i / 2], bk[i / 2], acc0, 0, 0, 0, 0, 0, 0);
                else
                    acc1 = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(rows.qa[1][i / 2], bk[i / 2], acc1, 0, 0, 0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < UPM; ++u) ea.unit(i * UPM + u, pa0, pa1, rows.wl);
                __builtin_amdgcn_sched_barrier(0);
            }
        } else {
            constexpr int NMF = 2 * G::KSTEPS, UPM = 32 / NMF;
            bf16x8 bk[G::KSTEPS];
#pragma unroll
            for (int s = 0; s < G::KSTEPS; ++s) bk[s] = as_bf16x8(*reinterpret_cast<const u32x4 *>(src + (ILV ? 32 : 16) * s));
#pragma unroll
            for (int i = 0; i < NMF; ++i) {
                if (i % 2 == 0)
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows.qa[0][i / 2], bk[i / 2], acc0, 0, 0, 0);
                else
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rows.qa[1][i / 2], bk[i / 2], acc1, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < UPM; ++u) ea.unit(i * UPM + u, pa0, pa1, rows.wl);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        sink(ea.finish(pks), pkey);
        pa0 = acc0;
        pa1 = acc1;
        pkey = key;
        pks = ksc;
    };

    // Sweep over nit tiles, the i-th being tile_of(i) (tile_of(nit) must name
    // a tile past the last key); the i-th tile's blocks carry the keys
    // i*KT + 32*cb + lane%32.  VM is the number of global memory operations
    // that `sink` issues per call.
    auto sweep = [&](int nit, auto tile_of, auto &sink, auto vm) {
        constexpr int VM = decltype(vm)::value;
        if constexpr (DMA) {
            constexpr int RS = ROWB / 16;        // 16-byte slots per LDS row (row + 1 pad)
            constexpr int NDMA = KT * RS / 64;   // 1 KB direct loads per tile (rows)
            constexpr int MPW = (NDMA + WAVES_PREFILL - 1) / WAVES_PREFILL;
            static_assert(KT * RS % 64 == 0, "tile must fill whole direct loads");
            // lane l of load m fills slot 64m + l = chunk c of tile row r (pad
            // slots re-read chunk 0); rows past the last key read as zeros
            uint32_t goff[MPW];
#pragma unroll
            for (int i = 0; i < MPW; ++i) {
                const int slot = 64 * (wave + WAVES_PREFILL * i) + lane;
                const int row = slot / RS, c = slot - row * RS;
                goff[i] = (uint32_t)(row * a.k_st + (c < RS - 1 ? 16 * c : 0));
            }
            auto gather = [&](int tile, uint8_t *dst) {
                const int64_t key0 = (int64_t)tile * KT;
                const int64_t rem = n_keys - key0;
                const int nk = rem < KT ? (int)rem : KT;  // keys of this tile
                const uint8_t *tbase = kb + key0 * a.k_st;
                const uint32_t bytes = (uint32_t)(nk * a.k_st);
#pragma unroll
                for (int i = 0; i < MPW; ++i) {
                    const int m = wave + WAVES_PREFILL * i;
                    if (m < NDMA) buffer_load_to_lds16(tbase, bytes, goff[i], dst + 1024 * m);
                }
                if constexpr (Q8) {
                    // the tile's KT key scales (4 per lane), by the last wave
                    if (wave == WAVES_PREFILL - 1 && lane < KT / 4)
                        buffer_load_to_lds16(a.k_scale + b * a.ks_sb + key0, (uint32_t)(nk * 4), 16 * lane,
                                             dst + KT * ROWB);
                }
            };
            auto step = [&](int it, const uint8_t *tb, uint8_t *nb) {
                if (it + 1 < nit) gather(tile_of(it + 1), nb);
#pragma unroll
                for (int cb = 0; cb < KT / 32; ++cb) {
                    const float ksc = Q8 ? *reinterpret_cast<const float *>(tb + KT * ROWB + 4 * (cb * 32 + l32)) : 1.f;
                    block(tb, cb, ksc, it * KT + cb * 32 + l32, sink);
                }
                // this wave's loads into nb have landed (only the sink's
                // stores issued after them may still be in flight), then all
                // waves' have
                wait_vmcnt<(KT / 32) * VM>();
                lds_barrier();
            };
            gather(tile_of(0), sk0);
            wait_vmcnt<0>();
            lds_barrier();
            for (int it = 0; it < nit; it += 2) {
                step(it, sk0, sk1);
                if (it + 1 >= nit) break;
                step(it + 1, sk1, sk0);
            }
        } else {
            // 16-byte chunks of one tile as read from memory: D/16 per key
            constexpr int SRC_CHUNK_KEY = D / 16;
            constexpr int SRC_CHUNKS = KT * SRC_CHUNK_KEY;
            constexpr int CPT = (SRC_CHUNKS + NT - 1) / NT;
            u32x4 pf[CPT];
            float pfs = 1.f;
            // range-checked buffer loads: keys past the last one (and chunks
            // past the tile) read as zeros without a branch, so the compiler
            // can count the loads in flight exactly (a key's zero scale is
            // never used)
            auto fetch = [&](int tile) {
                const int64_t key0 = (int64_t)tile * KT;
                const int64_t rem = n_keys - key0;
                const int nk = rem <= 0 ? 0 : (rem < KT ? (int)rem : KT);  // keys of this tile (0 past the end)
                const uint8_t *tbase = kb + key0 * a.k_st;
                const uint32_t bytes = (uint32_t)(nk * a.k_st);
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int c = tid + i * NT;
                    const int kk = c / SRC_CHUNK_KEY, part = c % SRC_CHUNK_KEY;
                    const uint32_t off = c < SRC_CHUNKS ? (uint32_t)(kk * a.k_st + part * 16) : bytes;
                    pf[i] = ld16_ranged(tbase, bytes, off);
                }
                pfs = ld4_ranged(a.k_scale + b * a.ks_sb + key0, (uint32_t)(nk * 4), tid < KT ? 4 * tid : (uint32_t)(nk * 4));
            };
            auto stash = [&](uint8_t *dst, int buf) {
#pragma unroll
                for (int i = 0; i < CPT; ++i) {
                    const int c = tid + i * NT;
                    if (c >= SRC_CHUNKS) break;
                    const int kk = c / SRC_CHUNK_KEY, part = c % SRC_CHUNK_KEY;
                    uint8_t *row = dst + kk * ROWB;
                    // 16 fp8 bytes -> 16 bf16 (32 bytes)
                    u32x2 lo0 = fp8x4_to_bf16x4(pf[i].x), lo1 = fp8x4_to_bf16x4(pf[i].y);
                    u32x2 hi0 = fp8x4_to_bf16x4(pf[i].z), hi1 = fp8x4_to_bf16x4(pf[i].w);
                    st16(row + part * 32, u32x4{lo0.x, lo0.y, lo1.x, lo1.y});
                    st16(row + part * 32 + 16, u32x4{hi0.x, hi0.y, hi1.x, hi1.y});
                }
                if (tid < KT) ssc[buf][tid] = pfs;
            };
            fetch(tile_of(0));
            stash(sk0, 0);
            __syncthreads();
            // (the tile after the last is fetched and stashed too -- as
            // zeros, into the buffer nobody reads any more -- so the loop body
            // has no branch around its loads and the compiler's wait counts
            // stay exact)
            for (int it = 0; it < nit; ++it) {
                const int buf = it & 1;
                fetch(tile_of(it + 1));
#pragma unroll
                for (int cb = 0; cb < KT / 32; ++cb)
                    block(buf ? sk1 : sk0, cb, ssc[buf][cb * 32 + l32], it * KT + cb * 32 + l32, sink);
                stash(buf ? sk0 : sk1, buf ^ 1);
                __syncthreads();
            }
        }
        sink(epi_reduce<H>(pa0, pa1, rows.wl, pks), pkey);
        pkey = -1;
        pa0 = f32x16{0};
        pa1 = f32x16{0};
    };
    auto all_tiles = [](int i) { return i; };

    if constexpr (!FUSE) {
        // (columns past the last key are not stored: a tile may reach
        // beyond the row stride)
        auto store_sink = [&](const Part<H> &pp, int key) {
            epi_store<H>(pp, rs, key >= 0 && key < n_keys, tq0, key, lane);
        };
        sweep(ntiles, all_tiles, store_sink, std::integral_constant<int, SPB>{});
    } else {
        // the lanes holding query q's reduced scores (one half of the wave)
        auto mine = [&](int q) { return QPW == 1 ? g == 0 : (q < QPW / 2) == (g == 0); };
        float tau[QPW];
#pragma unroll
        for (int q = 0; q < QPW; ++q) tau[q] = -__builtin_inff();
        if (n_keys > FUSE_CAP) {
            const int64_t n_min = a.q_pos0 + t0 + 1;
            const int nts = (int)(n_min / KT);  // whole tiles below every row's position
            // sampled tiles: enough for about 24 sampled scores at or above
            // each row's k-th largest, at least 4, at most NS (the LDS share)
            const int64_t want = (24 * n_min + (int64_t)a.top_k * KT - 1) / ((int64_t)a.top_k * KT);
            const int ns = (int)(want < 4 ? 4 : (want > NS ? NS : want));
            auto sample_tiles = [&](int i) { return i < ns ? (int)((int64_t)i * nts / ns) : ntiles; };
            auto sample_sink = [&](const Part<H> &pp, int key) {
                if (key < 0) return;
#pragma unroll
                for (int q = 0; q < QPW; ++q)
                    if (mine(q)) samp[(wave * QPW + q) * SPQ + key] = (uint16_t)(__float_as_uint(pp.v[q]) >> 16);
            };
            sweep(ns, sample_tiles, sample_sink, std::integral_constant<int, 0>{});
            // each wave reads only the samples it wrote
            const int nsk = ns * KT;  // sampled keys per row
#pragma unroll
            for (int q = 0; q < QPW; ++q) {
                if (tq0 + q >= a.T_q) break;
                const float n = (float)(a.q_pos0 + tq0 + q + 1);
                const float mu = (float)nsk * (float)a.top_k / n;
                float r = ceilf(mu + 4.5f * sqrtf(mu) + 2.f);
                r = fminf(fmaxf(r, 1.f), (float)nsk);
                tau[q] = sample_threshold<SPQ>(samp + (wave * QPW + q) * SPQ, nsk, (int)r, lane);
            }
        }
        constexpr uint32_t CAPB = FUSE_CAP * 8;
        uint32_t plim[QPW];
        int cnt[QPW];
#pragma unroll
        for (int q = 0; q < QPW; ++q) {
            // the row's last causal key (as unsigned, the key -1 before the
            // first block lies above it); rows past T_q pass nothing
            const bool row_ok = tq0 + q < a.T_q;
            plim[q] = row_ok ? (uint32_t)(a.q_pos0 + tq0 + q) : 0u;
            if (!row_ok) tau[q] = __builtin_inff();
            cnt[q] = 0;
        }
        auto filter_sink = [&](const Part<H> &pp, int key) {
#pragma unroll
            for (int q = 0; q < QPW; ++q) {
                // (bitwise ands: no short-circuit branches in the loop)
                const bool pass = mine(q) & ((uint32_t)key <= plim[q]) & (pp.v[q] >= tau[q]);
                const uint64_t m = ballot(pass);
                const uint32_t off = pass ? (uint32_t)(cnt[q] + lanes_below(m)) * 8u : CAPB;
                uint32_t *base = a.cand + ((int64_t)b * a.T_q + tq0 + q) * (2 * FUSE_CAP);
                store_b64_ranged(base, CAPB, off, u32x2{__float_as_uint(pp.v[q]), (uint32_t)key});
                cnt[q] = min(cnt[q] + (int)__popcll(m), FUSE_CAP + 1);  // saturates past the slots
            }
        };
        sweep(ntiles, all_tiles, filter_sink, std::integral_constant<int, SPB>{});
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < QPW; ++q) {
                const int t = tq0 + q;
                if (t >= a.T_q) break;
                const int32_t id = b * a.T_q + t;
                a.ccnt[id] = cnt[q];
                if (fused_row_bad(cnt[q], a.q_pos0 + t + 1, a.top_k)) {
                    const int slot = atomicAdd(a.rcount, 1);
                    if (slot < a.rmax) a.rlist[slot] = id;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Split-key variant for few query rows (decode): a workgroup takes one group
// of 64/H query rows and a contiguous key range; its 4 waves stride over the
// 32-key blocks of that range, each block read from HBM in whole key rows
// (load i of a block gives lane l the 16-byte chunk l % CPR of key
// RPL*i + l / CPR: every load instruction covers RPL consecutive rows, with
// the non-temporal hint, as the keys are read once) two blocks ahead of the
// compute.  A wave turns a block into its B fragments through its own LDS
// tile (row-major, rows padded by 16 bytes: conflict-free in both
// directions), so no barrier is needed.  (Loads that give each lane its own
// key directly touch 32 keys' cache lines per instruction instead of RPL
// rows': 12 % slower at 131K keys.)
// ---------------------------------------------------------------------------
template <int H, int D, int F, int NB, int OCC>
__global__ __launch_bounds__(WAVES_SPLIT * 64) __attribute__((amdgpu_waves_per_eu(OCC))) void score_splitkey_kernel(ScoreArgs a)
{
    using G = KeyGeom<D>;
    constexpr bool Q8 = F == F_QK8;
    constexpr bool K8 = F != F_BF16;
    constexpr bool ILV = !K8;  // interleaved d map
    constexpr int QPW = 64 / H;
    // per lane: G::HALF key elements = HALF*2 bytes (bf16) or HALF bytes (fp8)
    constexpr int NLD = K8 ? G::HALF / 16 : G::HALF / 8;  // 16-byte loads per lane per block
    constexpr int ROWK = K8 ? D : 2 * D;                   // bytes per key row
    constexpr int CPR = ROWK / 16;                         // 16-byte chunks per key row
    constexpr int RPL = 64 / CPR;                          // key rows per load instruction
    constexpr int ROWP = ROWK + 16;                        // LDS bytes per key row (padded)
    static_assert(NLD * RPL == 32, "a block is NLD whole-row loads");
    __shared__ __attribute__((aligned(16))) uint8_t tr[WAVES_SPLIT][32 * ROWP];

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    int b = blockIdx.z;
    int tq0 = blockIdx.y * QPW;
    if (a.rlist) {
        // rescoring listed rows: entry blockIdx.y names the row (its group)
        if ((int)blockIdx.y >= min(*a.rcount, a.rmax)) return;
        const int id = a.rlist[blockIdx.y];
        b = id / a.T_q;
        const int t = id - b * a.T_q;
        tq0 = t - t % QPW;
    }
    const int64_t n_keys = a.q_pos0 + min(a.T_q, tq0 + QPW);
    const int64_t key_lo = (int64_t)blockIdx.x * a.key_split;
    const int64_t key_hi = min<int64_t>(n_keys, key_lo + a.key_split);
    if (key_lo >= key_hi) return;
    const int nblk = (int)((key_hi - key_lo + 31) / 32);

    typename std::conditional<Q8, WaveRows8<H, D>, WaveRows<H, D, ILV>>::type rows;
    rows.load(a, b, tq0, lane);
    const uint8_t *kb = a.k + b * a.k_sb;
    float *Sb = a.S + (int64_t)b * a.T_q * a.ld;
    const RowSpan rs{Sb + (int64_t)tq0 * a.ld, (uint32_t)((min(a.T_q, tq0 + QPW) - tq0) * a.ld * 4), a.ld, tq0};

    // NB register buffers: the blocks NB-1 .. 1 steps ahead are in flight
    // while the current one computes (the loop is unrolled by NB, so the
    // buffers rotate by compile-time index, without copies)
    u32x4 r[NB][NLD];
    float sc[NB];
    // keys key_lo .. key_hi-1 through range-checked buffer loads: blocks and
    // keys past the range read as zeros without a branch
    const uint8_t *kr = kb + key_lo * a.k_st;
    const uint32_t kr_bytes = (uint32_t)((key_hi - key_lo) * a.k_st);
    const float *sr = K8 ? a.k_scale + b * a.ks_sb + key_lo : nullptr;
    const uint32_t sr_bytes = (uint32_t)((key_hi - key_lo) * 4);
    // Each buffer keeps its own running byte offsets (advanced by three
    // blocks per use), so the load addresses live in registers of their own
    // and never share one with a load still in flight.
    const uint32_t kstride = (uint32_t)(NB * WAVES_SPLIT * 32) * (uint32_t)a.k_st;
    const uint32_t sstride = NB * WAVES_SPLIT * 32 * 4;
    const uint32_t rstep = (uint32_t)RPL * (uint32_t)a.k_st;  // bytes between a block's loads
    auto fetch = [&](uint32_t &koff, uint32_t &soff, u32x4 (&rb)[NLD], float &sb) {
#pragma unroll
        for (int i = 0; i < NLD; ++i) rb[i] = ld16_ranged_nt(kr, kr_bytes, koff + rstep * i);
        if constexpr (K8) sb = ld4_ranged(sr, sr_bytes, soff);
        koff += kstride;
        soff += sstride;
    };
    // the block's chunks through this wave's LDS tile: written as loaded,
    // read back as this lane's key (l32) and k-slot chunks -- chunk 2i + g
    // (bf16, the interleaved map) or g*CPR/2 + i (fp8, split halves)
    uint8_t *tw = tr[wave];
    auto to_lanes = [&](const u32x4 (&ld)[NLD], u32x4 (&x)[NLD]) {
        uint8_t *wp = tw + (lane / CPR) * ROWP + 16 * (lane % CPR);
#pragma unroll
        for (int i = 0; i < NLD; ++i) st16(wp + RPL * ROWP * i, ld[i]);
        const uint8_t *rp = tw + l32 * ROWP;
#pragma unroll
        for (int i = 0; i < NLD; ++i) x[i] = ld16(rp + 16 * (ILV ? 2 * i + g : g * (CPR / 2) + i));
    };
    auto step = [&](int blk, const u32x4 (&ld)[NLD], float cs, u32x4 (&ahead)[NLD], float &as, uint32_t &koff,
                    uint32_t &soff) {
        fetch(koff, soff, ahead, as);
        u32x4 cur[NLD];
        to_lanes(ld, cur);
        f32x16 acc0, acc1;
        if constexpr (Q8) {
            i32x8 bk[G::KSTEPS8];
#pragma unroll
            for (int s = 0; s < G::KSTEPS8; ++s) {
                const u32x4 lo = cur[2 * s], hi = cur[2 * s + 1];
                bk[s] = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
            mfma_block8<D>(rows.qa, bk, acc0, acc1);
        } else {
            bf16x8 bk[G::KSTEPS];
            if constexpr (K8) {
#pragma unroll
                for (int i = 0; i < NLD; ++i) {
                    u32x2 p0 = fp8x4_to_bf16x4(cur[i].x), p1 = fp8x4_to_bf16x4(cur[i].y);
                    u32x2 p2 = fp8x4_to_bf16x4(cur[i].z), p3 = fp8x4_to_bf16x4(cur[i].w);
                    bk[2 * i] = as_bf16x8(u32x4{p0.x, p0.y, p1.x, p1.y});
                    bk[2 * i + 1] = as_bf16x8(u32x4{p2.x, p2.y, p3.x, p3.y});
                }
            } else {
#pragma unroll
                for (int i = 0; i < NLD; ++i) bk[i] = as_bf16x8(cur[i]);
            }
            mfma_block<D>(rows.qa, bk, acc0, acc1);
        }
        const int64_t key = key_lo + (int64_t)blk * 32 + l32;
        epi_store<H>(epi_reduce<H>(acc0, acc1, rows.wl, cs), rs, key < key_hi, tq0, (int)key, lane);
    };

    int blk = wave;
    const uint32_t lbase = (uint32_t)(lane / CPR) * (uint32_t)a.k_st + 16u * (uint32_t)(lane % CPR);
    // each buffer keeps its own running byte offsets (advanced by NB blocks
    // per use), so the load addresses live in registers of their own and
    // never share one with a load still in flight
    uint32_t ko[NB], so[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        ko[u] = (uint32_t)((blk + u * WAVES_SPLIT) * 32) * (uint32_t)a.k_st + lbase;
        so[u] = (uint32_t)((blk + u * WAVES_SPLIT) * 32 + l32) * 4;
        sc[u] = 1.f;
    }
#pragma unroll
    for (int u = 0; u < NB - 1; ++u) fetch(ko[u], so[u], r[u], sc[u]);
    for (; blk < nblk; blk += NB * WAVES_SPLIT) {
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            if (u > 0 && blk + u * WAVES_SPLIT >= nblk) break;
            const int nx = (u + NB - 1) % NB;  // the buffer consumed by the previous step
            step(blk + u * WAVES_SPLIT, r[u], sc[u], r[nx], sc[nx], ko[nx], so[nx]);
        }
    }
}

template <int H, int D, int F>
hipError_t launch_score_hd(const ScoreArgs &a, bool split, hipStream_t st)
{
    constexpr int QPW = 64 / H;
    if (!split) {
        constexpr int QPB = WAVES_PREFILL * QPW;
        dim3 grid((a.T_q + QPB - 1) / QPB, a.B);
        if constexpr (H >= 16) {
            if (a.fuse) {
                hipLaunchKernelGGL((score_prefill_kernel<H, D, F, true>), grid, dim3(WAVES_PREFILL * 64), 0, st, a);
                return hipGetLastError();
            }
        }
        if (a.fuse) return hipErrorInvalidValue;
        hipLaunchKernelGGL((score_prefill_kernel<H, D, F, false>), grid, dim3(WAVES_PREFILL * 64), 0, st, a);
    } else {
        if (a.fuse || a.redo) return hipErrorInvalidValue;
        const int64_t n_keys = a.q_pos0 + a.T_q;
        dim3 grid((unsigned)((n_keys + a.key_split - 1) / a.key_split), (a.T_q + QPW - 1) / QPW, a.B);
        if (a.rlist) grid = dim3(grid.x, a.rmax, 1);
        if constexpr (F == F_BF16)
            hipLaunchKernelGGL((score_splitkey_kernel<H, D, F, SPLIT_NB_BF16, SPLIT_OCC_BF16>), grid, dim3(WAVES_SPLIT * 64), 0, st, a);
        else
            hipLaunchKernelGGL((score_splitkey_kernel<H, D, F, SPLIT_NB_F8, SPLIT_OCC_F8>), grid, dim3(WAVES_SPLIT * 64), 0, st, a);
    }
    return hipGetLastError();
}

template <int H, int D>
hipError_t launch_score_f(const ScoreArgs &a, bool split, hipStream_t st)
{
    if (a.q8) return launch_score_hd<H, D, F_QK8>(a, split, st);
    if (a.fp8) return launch_score_hd<H, D, F_K8>(a, split, st);
    return launch_score_hd<H, D, F_BF16>(a, split, st);
}

template <int H>
hipError_t launch_score_h(const ScoreArgs &a, bool split, hipStream_t st)
{
    if (a.D == 128) return launch_score_f<H, 128>(a, split, st);
    return launch_score_f<H, 64>(a, split, st);
}

}  // namespace

// Heuristic: the LDS-staged prefill kernel when there are enough query rows
// to fill the chip, the split-key kernel otherwise.  Both give identical bits.
bool score_use_split(const ScoreArgs &a)
{
    const int qpb = WAVES_PREFILL * (64 / a.H);
    const int64_t blocks = (int64_t)a.B * ((a.T_q + qpb - 1) / qpb);
    return blocks < 256 && (a.q_pos0 + a.T_q) >= 4096;
}

bool score_can_fuse(const ScoreArgs &a)
{
    // only when some row is longer than its candidate slots: shorter rows
    // would keep every score, as 8-byte pairs against 4-byte score rows
    return a.H >= 16 && !score_use_split(a) && a.q_pos0 + a.T_q > FUSE_CAP;
}

int score_key_range(int64_t ks, int64_t k_st_bytes)
{
    // the keys of one workgroup are read through a buffer resource with
    // 32-bit offsets: at most 2^31 - 1 bytes (a multiple of 32 keys; the
    // key stride is below 16 MiB, so at least 128 keys)
    const int64_t lim = ((((int64_t)1 << 31) - 1) / (k_st_bytes > 0 ? k_st_bytes : 1)) / 32 * 32;
    return (int)(ks < lim ? ks : lim);
}

int score_key_split(const ScoreArgs &a)
{
    // aim for >= ~512 workgroups (two per CU, one round: 4-5 % faster at
    // 131K and 1M keys than two rounds of 1024, no better at 2048 or 4096);
    // keep ranges a multiple of 256 keys
    const int64_t n_keys = a.q_pos0 + a.T_q;
    const int64_t groups = (int64_t)a.B * ((a.T_q + 64 / a.H - 1) / (64 / a.H));
    int64_t splits = (SPLIT_WGS + groups - 1) / groups;
    int64_t ks = (n_keys + splits - 1) / splits;
    ks = ((ks + 255) / 256) * 256;
    if (ks < 512) ks = 512;
    return score_key_range(ks, a.k_st);
}

namespace {
__global__ void zero_i32_kernel(int32_t *p) { *p = 0; }
}  // namespace

hipError_t launch_zero_i32(int32_t *p, hipStream_t st)
{
    hipLaunchKernelGGL(zero_i32_kernel, dim3(1), dim3(1), 0, st, p);
    return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, hipStream_t st)
{
    const bool split = a.rlist && !a.fuse ? true : score_use_split(a);
    switch (a.H) {
    case 4: return launch_score_h<4>(a, split, st);
    case 8: return launch_score_h<8>(a, split, st);
    case 16: return launch_score_h<16>(a, split, st);
    case 32: return launch_score_h<32>(a, split, st);
    case 64: return launch_score_h<64>(a, split, st);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace lcsi
