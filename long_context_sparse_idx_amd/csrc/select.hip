// Per-row top-k selection for gfx950 (the second half of the indexer's
// "dot product + top-k": IndexShare term page (earlyterms.com), opening
// definition; each token keeps its top-k positions: IndexShare explainer
// (yun88.com), section on the hidden indexer cost).
//
// Row p holds n = p + 1 fp32 scores.  Output: the min(k, n) positions with
// the largest scores, ties to the lower position, in ascending position
// order, padded with -1 to k entries.
//
// Scores are compared through an order-preserving uint32 key (-0 folded onto
// +0), so selection is exact integer work: a radix select with 8-bit digits
// (LDS histograms) finds the k-th largest key K* and how many entries equal
// to K* are taken; a stable, wave-ordered compaction then writes every entry
// with key > K* and the first `need` entries with key == K*.
//
// One 512-thread workgroup per row, three paths (after a fused score pass,
// rows whose candidate count is usable select from their candidates
// instead):
//  A  n <= 16384: the whole row's keys sit in LDS; select there.
//  B  longer rows: 8192 sampled scores (32 evenly spaced runs of 256) give
//     a threshold tau that somewhat more than k entries are expected to
//     reach (four standard deviations of the sampling error above k); one
//     streaming pass keeps every entry with key >= tau in per-wave ordered
//     LDS lists, and the exact select runs on those.  If fewer than k
//     entries pass, or a list overflows, the row falls back to C.  The
//     result never depends on the sample, only the cost does.
//  C  exact radix select and compaction streaming the row from memory.
//
// Few long rows (decode: a handful of sequences, each with up to a million
// scores) would leave most of the chip idle with one workgroup per row, so
// they take a two-kernel form of path B: many workgroups per row each find
// the row's sampled threshold (the same in all of them) and filter one
// segment into a per-segment candidate list in the workspace (ordered); one
// workgroup per row gathers the lists (ascending positions, segment after
// segment) and runs the exact select on them -- or path C when a segment
// overflowed or fewer than k entries passed.
#include "device_common.h"
#include "kernels.h"

namespace lcsi {

namespace {

constexpr int NT = 512;
constexpr int NW = NT / 64;
constexpr int NLDS = 16384;       // path A limit
constexpr int CAPW = 1024;        // candidate slots per wave (path B)
constexpr int NSB = 32;           // sample runs
constexpr int SBL = 256;          // run length
constexpr int NSAMP = NSB * SBL;
constexpr int NSUB = 4;           // histogram copies (waves w and w+4k share one)

struct Shared {
    union {
        uint32_t keys[NLDS];                     // path A
        struct {
            uint32_t key[NW * CAPW];
            int32_t idx[NW * CAPW];
        } cand;                                  // path B candidates
    } u;
    uint32_t hist[3][NSUB][256] __attribute__((aligned(16)));  // radix histograms, three in rotation
    int wcnt[NW];
    int wgt[NW];
    int wtie[NW];
    int nsmall;
    uint32_t small[64];           // the keys of a small final bin (offsets)
    uint32_t wmin[NW], wmax[NW];  // per-wave key range, written while filling LDS
};

// ---- wave-wide sums, scans and ranges through DPP lane moves and
// v_readlane (no LDS traffic).  Rows are the four 16-lane quarters of a
// wave; a DPP source lane outside the row reads as 0.
template <int CTRL>
__device__ __forceinline__ int dpp(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
constexpr int DPP_QUAD_XOR1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_XOR2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int DPP_ROW_SHL = 0x100;   // + n: lane i takes lane i + n of its row
constexpr int DPP_ROW_SHR = 0x110;   // + n: lane i takes lane i - n of its row
constexpr int DPP_ROW_ROR = 0x120;   // + n: rotate within the row

__device__ __forceinline__ int wave_sum(int v)
{
    v += dpp<DPP_QUAD_XOR1>(v);
    v += dpp<DPP_QUAD_XOR2>(v);
    v += dpp<DPP_ROW_ROR + 4>(v);
    v += dpp<DPP_ROW_ROR + 8>(v);  // every lane: its row's sum
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ uint32_t wave_min(uint32_t v)
{
    v = min(v, (uint32_t)dpp<DPP_QUAD_XOR1>((int)v));
    v = min(v, (uint32_t)dpp<DPP_QUAD_XOR2>((int)v));
    v = min(v, (uint32_t)dpp<DPP_ROW_ROR + 4>((int)v));
    v = min(v, (uint32_t)dpp<DPP_ROW_ROR + 8>((int)v));
    const uint32_t a = min((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = min((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return min(a, b);
}

__device__ __forceinline__ uint32_t wave_max(uint32_t v)
{
    v = max(v, (uint32_t)dpp<DPP_QUAD_XOR1>((int)v));
    v = max(v, (uint32_t)dpp<DPP_QUAD_XOR2>((int)v));
    v = max(v, (uint32_t)dpp<DPP_ROW_ROR + 4>((int)v));
    v = max(v, (uint32_t)dpp<DPP_ROW_ROR + 8>((int)v));
    const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
    const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
    return max(a, b);
}

// Inclusive suffix sum over lanes >= this one.
__device__ __forceinline__ int wave_suffix_sum(int v)
{
    v += dpp<DPP_ROW_SHL + 1>(v);
    v += dpp<DPP_ROW_SHL + 2>(v);
    v += dpp<DPP_ROW_SHL + 4>(v);
    v += dpp<DPP_ROW_SHL + 8>(v);  // suffix within the row; lane 16 r: row r's sum
    const int r1 = __builtin_amdgcn_readlane(v, 16), r2 = __builtin_amdgcn_readlane(v, 32),
              r3 = __builtin_amdgcn_readlane(v, 48);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row < 1 ? r1 : 0) + (row < 2 ? r2 : 0) + (row < 3 ? r3 : 0);
}

// Inclusive prefix sum over lanes <= this one.
__device__ __forceinline__ int wave_prefix_sum(int v)
{
    v += dpp<DPP_ROW_SHR + 1>(v);
    v += dpp<DPP_ROW_SHR + 2>(v);
    v += dpp<DPP_ROW_SHR + 4>(v);
    v += dpp<DPP_ROW_SHR + 8>(v);  // prefix within the row; lane 16 r + 15: row r's sum
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = (threadIdx.x & 63) >> 4;
    return v + (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
}

// ---- element visitors: each thread calls f(key) for its share ------------

struct LdsKeys {
    const uint32_t *keys;
    int n;
    template <class F> __device__ void visit(F f) const
    {
        for (int i = threadIdx.x; i < n; i += NT) f(keys[i]);
    }
};

// Keys held in registers: IT keys per thread, key u valid where bit u of
// `valid` is set.
template <int IT>
struct RegKeys {
    uint32_t k[IT];
    uint32_t valid;
    template <class F> __device__ __forceinline__ void visit(F f) const
    {
#pragma unroll
        for (int u = 0; u < IT; ++u)
            if ((valid >> u) & 1u) f(k[u]);
    }
};

struct Candidates {
    const Shared *sh;
    template <class F> __device__ void visit(F f) const
    {
        const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
        const int c = sh->wcnt[w];
        for (int j = lane; j < c; j += 64) f(sh->u.cand.key[w * CAPW + j]);
    }
};

struct GlobalRow {
    const float *row;
    int64_t n;
    template <class F> __device__ void visit(F f) const
    {
        for (int64_t i = 4 * (int64_t)threadIdx.x; i < n; i += 4 * NT) {
            const f32x4 v = *reinterpret_cast<const f32x4 *>(row + i);
            f(order_key(v.x));
            if (i + 1 < n) f(order_key(v.y));
            if (i + 2 < n) f(order_key(v.z));
            if (i + 3 < n) f(order_key(v.w));
        }
    }
};

// Candidates of a fused score pass: (score bits, position) pairs in
// ascending position order.
struct GlobalPairs {
    const uint32_t *p;
    int n;
    template <class F> __device__ void visit(F f) const
    {
        for (int i = threadIdx.x; i < n; i += NT) f(order_key(__uint_as_float(p[2 * i])));
    }
};

// Find the rank-th largest key (rank >= 1, at most the number of visited
// keys).  Returns that key and the number of entries equal to it that
// belong to the top `rank` -- the same in every thread.
//
// The 8-bit digit passes run on the offset key - kmin (kmin, kmax: the
// smallest and largest key), starting at the highest bit of the range
// kmax - kmin, so the first 256 bins span the keys actually present (scores
// of one row share sign and exponent bits, and a digit over those bits
// would put nearly every key into one or two bins).  A pass is one
// histogram (LDS atomics into one of NSUB copies by wave), one barrier, and
// the bin search, which every wave does for itself on the shared counts.
// The histograms rotate over three buffers: the one a pass fills was last
// read two passes earlier, and the pass before clears it during its visit.
// When at most 64 keys are left in the chosen bin they are collected and
// ranked directly instead of further passes.
// resolve < 32 stops once that many offset bits from the top are fixed and
// at most max_ge keys lie at or above the current bin: the key returned is
// then kmin + the offset prefix with the lower bits cleared -- a lower
// bound of the rank-th key that at least `rank` and at most max_ge keys
// reach (used for sampled thresholds, where only a bound is needed).
// ranged = true: the caller has written every wave's key range with
// wave_range and called radix_prepare, both before a barrier.  Two calls
// must be separated by a barrier (the second clears what the first reads).
struct Kth {
    uint32_t key;
    int rem;
};

// The smallest and largest of a thread's keys (kmn, kmx) reduced over the
// wave into its slot of sh.wmin / sh.wmax (every wave writes its slot; a
// wave without keys writes the empty range).
__device__ __forceinline__ void wave_range(Shared &sh, uint32_t kmn, uint32_t kmx)
{
    kmn = wave_min(kmn);
    kmx = wave_max(kmx);
    if ((threadIdx.x & 63) == 0) {
        sh.wmin[threadIdx.x >> 6] = kmn;
        sh.wmax[threadIdx.x >> 6] = kmx;
    }
}

// Clears the first pass's histograms and the small-bin count.
__device__ __forceinline__ void radix_prepare(Shared &sh)
{
    for (int i = threadIdx.x; i < NSUB * 256; i += NT) (&sh.hist[0][0][0])[i] = 0;
    if (threadIdx.x == 0) sh.nsmall = 0;
}

template <class Src>
__device__ Kth radix_find(Shared &sh, const Src &src, int rank, int resolve = 32, int max_ge = 0x7FFFFFFF,
                          bool ranged = false)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    if (!ranged) {
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        src.visit([&](uint32_t key) {
            kmn = min(kmn, key);
            kmx = max(kmx, key);
        });
        wave_range(sh, kmn, kmx);
        radix_prepare(sh);
        __syncthreads();
    }
    uint32_t kmin = 0xFFFFFFFFu, kmax = 0u;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        kmin = min(kmin, sh.wmin[v]);
        kmax = max(kmax, sh.wmax[v]);
    }
    const uint32_t range = kmax - kmin;
    if (range == 0) return {kmin, rank};  // all keys equal: the rank-th is that key
    const int msb = 31 - __builtin_clz(range);
    uint32_t mask = msb == 31 ? 0u : ~((2u << msb) - 1u);  // offset bits already fixed (all zero)
    uint32_t prefix = 0;                                    // fixed offset bits
    int rem = rank;
    int hi = msb;  // highest bit of the next digit
#pragma unroll 1
    for (int p = 0;; ++p) {
        const int shift = hi >= 7 ? hi - 7 : 0;
        const uint32_t dmask = (2u << (hi - shift)) - 1u;  // digit width hi-shift+1 <= 8 bits
        const int b = p % 3;
        uint32_t *hw = sh.hist[b][w % NSUB];
        for (int i = tid; i < NSUB * 256; i += NT) (&sh.hist[(p + 1) % 3][0][0])[i] = 0;
        src.visit([&](uint32_t key) {
            const uint32_t off = key - kmin;
            if ((off & mask) == prefix) atomicAdd(&hw[(off >> shift) & dmask], 1u);
        });
        __syncthreads();
        // bin search (every wave): lane l owns bins 4l .. 4l+3
        uint32_t c[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int h = 0; h < NSUB; ++h) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(&sh.hist[b][h][4 * lane]);
            c[0] += v.x;
            c[1] += v.y;
            c[2] += v.z;
            c[3] += v.w;
        }
        const int tot = (int)(c[0] + c[1] + c[2] + c[3]);
        const int suf = wave_suffix_sum(tot);  // over lanes >= this one
        const int above = suf - tot;
        const bool found = above < rem && rem <= suf;  // exactly one lane
        uint32_t f_prefix = 0;
        int f_rem = 0, f_ge = 0, f_c = 0;
        if (found) {
            int acc = above;
            for (int e = 3; e >= 0; --e) {
                if (acc + (int)c[e] >= rem) {
                    f_prefix = prefix | ((uint32_t)(4 * lane + e) << shift);
                    f_rem = rem - acc;
                    f_ge = (rank - rem) + acc + (int)c[e];  // keys at or above this bin
                    f_c = (int)c[e];
                    break;
                }
                acc += (int)c[e];
            }
        }
        const int fl = __ffsll((long long)ballot(found)) - 1;
        prefix = __builtin_amdgcn_readlane(f_prefix, fl);
        rem = __builtin_amdgcn_readlane(f_rem, fl);
        const int ge = __builtin_amdgcn_readlane(f_ge, fl);
        const int binc = __builtin_amdgcn_readlane(f_c, fl);
        mask |= dmask << shift;
        if (shift == 0 || (msb - shift + 1 >= resolve && ge <= max_ge)) break;
        if (resolve == 32 && binc == rem && prefix != 0) {
            // every key of the bin is taken: the keys above offset prefix - 1
            // (this bin and everything above it) are exactly the top `rank`,
            // so the threshold is prefix - 1 with no ties to count
            prefix -= 1;
            rem = 0;
            break;
        }
        if (resolve == 32 && binc <= 64) {
            // at most 64 keys left in the bin: collect them and rank them
            // directly -- the rem-th largest x has fewer than rem keys above
            // it and at least rem at or above it
            const uint32_t bmask = mask, bprefix = prefix;
            src.visit([&](uint32_t key) {
                const uint32_t off = key - kmin;
                if ((off & bmask) == bprefix) sh.small[atomicAdd(&sh.nsmall, 1)] = off;
            });
            __syncthreads();
            const uint32_t x = lane < binc ? sh.small[lane] : 0u;
            int gt = 0, geq = 0;
            for (int j = 0; j < binc; ++j) {  // (uniform; lane j's key read into a scalar)
                const uint32_t y = __builtin_amdgcn_readlane(x, j);
                gt += y > x;
                geq += y >= x;
            }
            const int f2 = __ffsll((long long)ballot(lane < binc && gt < rem && rem <= geq)) - 1;
            prefix = __builtin_amdgcn_readlane(x, f2);
            rem -= __builtin_amdgcn_readlane(gt, f2);
            break;
        }
        hi = shift - 1;
    }
    return {kmin + prefix, rem};
}

// Ordered compaction over per-wave segments visited in ascending position
// order.  Seg::get(w, j, key, pos) returns false past the end of segment w;
// Seg::len(w) is an upper bound on its length (a multiple of 64 not needed).
template <class Seg>
__device__ void emit(Shared &sh, const Seg &seg, int32_t *out, int k, Kth t)
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint32_t kth = t.key;
    const int need = t.rem;
    const int len = seg.len(w);
    int gt = 0, tie = 0;
    for (int j = lane; j < len; j += 64) {
        uint32_t key;
        int32_t pos;
        if (seg.get(w, j, key, pos)) {
            gt += key > kth;
            tie += key == kth;
        }
    }
    gt = wave_sum(gt);
    tie = wave_sum(tie);
    if (lane == 0) {
        sh.wgt[w] = gt;
        sh.wtie[w] = tie;
    }
    __syncthreads();
    int tie_off = 0, out_off = 0;
    for (int v = 0; v < w; ++v) {
        const int take = min(max(need - tie_off, 0), sh.wtie[v]);
        out_off += sh.wgt[v] + take;
        tie_off += sh.wtie[v];
    }
    for (int j0 = 0; j0 < len; j0 += 64) {
        uint32_t key = 0;
        int32_t pos = -1;
        const bool ok = seg.get(w, j0 + lane, key, pos);
        const bool is_tie = ok && key == kth;
        const uint64_t bt = ballot(is_tie);
        const bool sel = ok && (key > kth || (is_tie && tie_off + lanes_below(bt) < need));
        const uint64_t bs = ballot(sel);
        const int slot = out_off + lanes_below(bs);
        if (sel && slot < k) out[slot] = pos;
        tie_off += __popcll(bt);
        out_off += __popcll(bs);
    }
}

// The same compaction for keys held in registers: thread (w, lane) holds
// entries lane + 64 u (u = 0 .. IT-1) of wave w's run, the waves' runs
// follow one another, and every run is in ascending position order.
template <int IT>
__device__ void emit_regs(Shared &sh, const RegKeys<IT> &rk, const int32_t (&pos)[IT], int32_t *out, int k, Kth t)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t kth = t.key;
    const int need = t.rem;
    int gt = 0, tie = 0;
#pragma unroll
    for (int u = 0; u < IT; ++u)
        if ((rk.valid >> u) & 1u) {
            gt += rk.k[u] > kth;
            tie += rk.k[u] == kth;
        }
    gt = wave_sum(gt);
    tie = wave_sum(tie);
    if (lane == 0) {
        sh.wgt[w] = gt;
        sh.wtie[w] = tie;
    }
    __syncthreads();
    int tie_off = 0, out_off = 0;
    for (int v = 0; v < w; ++v) {
        const int take = min(max(need - tie_off, 0), sh.wtie[v]);
        out_off += sh.wgt[v] + take;
        tie_off += sh.wtie[v];
    }
#pragma unroll
    for (int u = 0; u < IT; ++u) {
        if (ballot((rk.valid >> u) != 0u) == 0) break;  // no lane has entries from slot u on
        const bool ok = (rk.valid >> u) & 1u;
        const bool is_tie = ok && rk.k[u] == kth;
        const uint64_t bt = ballot(is_tie);
        const bool sel = ok && (rk.k[u] > kth || (is_tie && tie_off + lanes_below(bt) < need));
        const uint64_t bs = ballot(sel);
        const int slot = out_off + lanes_below(bs);
        if (sel && slot < k) out[slot] = pos[u];
        tie_off += __popcll(bt);
        out_off += __popcll(bs);
    }
}

struct LdsSeg {
    const Shared *sh;
    int n, seg;
    __device__ int len(int w) const { return seg; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        const int i = w * seg + j;
        if (j >= seg || i >= n) return false;
        key = sh->u.keys[i];
        pos = i;
        return true;
    }
};

struct CandSeg {
    const Shared *sh;
    __device__ int len(int w) const { return sh->wcnt[w]; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        if (j >= sh->wcnt[w]) return false;
        key = sh->u.cand.key[w * CAPW + j];
        pos = sh->u.cand.idx[w * CAPW + j];
        return true;
    }
};

// Candidates stored contiguously in the LDS candidate arrays (ascending
// positions), cut into NW consecutive segments of `seg` entries.
struct LdsPairSeg {
    const Shared *sh;
    int n, seg;
    __device__ int len(int w) const { return seg; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        const int i = w * seg + j;
        if (j >= seg || i >= n) return false;
        key = sh->u.cand.key[i];
        pos = sh->u.cand.idx[i];
        return true;
    }
};

struct GlobalSeg {
    const float *row;
    int64_t n, seg;
    __device__ int len(int w) const { return (int)seg; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        const int64_t i = (int64_t)w * seg + j;
        if (j >= seg || i >= n) return false;
        key = order_key(row[i]);
        pos = (int32_t)i;
        return true;
    }
};

struct GlobalPairSeg {
    const uint32_t *p;
    int n, seg;
    __device__ int len(int w) const { return seg; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        const int i = w * seg + j;
        if (j >= seg || i >= n) return false;
        const u32x2 e = *reinterpret_cast<const u32x2 *>(p + 2 * i);
        key = order_key(__uint_as_float(e.x));
        pos = (int32_t)e.y;
        return true;
    }
};

// Exact top-k of a row from the c >= k candidates of a fused score pass
// (every score at or above the row's k-th largest is among them): in the
// per-wave LDS lists when they fit, as an LDS row when the candidates are
// the whole row (n <= NLDS), else streaming the pairs from memory.
__device__ void select_from_pairs(Shared &sh, const uint32_t *cp, int c, int64_t n, int32_t *out, int k)
{
    const int tid = threadIdx.x;
    const int seg = ((c + NW - 1) / NW + 63) / 64 * 64;
    if (c <= NW * CAPW) {
        // all loads of a thread issued before the first store (two pairs per
        // 16-byte range-checked load: pairs past the count read as zeros and
        // are not stored), the candidates kept contiguous in position order
        constexpr int IT = NW * CAPW / (2 * NT);
        u32x4 e[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) e[u] = ld16_ranged(cp, (uint32_t)c * 8u, 16u * (uint32_t)(tid + u * NT));
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int i = 2 * (tid + u * NT);
            if (i < c) {
                const uint32_t key = order_key(__uint_as_float(e[u].x));
                sh.u.cand.key[i] = key;
                sh.u.cand.idx[i] = (int32_t)e[u].y;
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
            if (i + 1 < c) {
                const uint32_t key = order_key(__uint_as_float(e[u].z));
                sh.u.cand.key[i + 1] = key;
                sh.u.cand.idx[i + 1] = (int32_t)e[u].w;
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
        }
        wave_range(sh, kmn, kmx);
        radix_prepare(sh);
        __syncthreads();
        const Kth t = radix_find(sh, LdsKeys{sh.u.cand.key, c}, k, 32, 0x7FFFFFFF, true);
        emit(sh, LdsPairSeg{&sh, c, seg}, out, k, t);
        return;
    }
    if (c == n && n <= NLDS) {
        // every score passed: the candidates are the row, positions 0 .. n-1
        constexpr int IT = NLDS / (2 * NT);
        u32x4 e[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) e[u] = ld16_ranged(cp, (uint32_t)c * 8u, 16u * (uint32_t)(tid + u * NT));
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int i = 2 * (tid + u * NT);
            if (i < c) {
                const uint32_t key = order_key(__uint_as_float(e[u].x));
                sh.u.keys[i] = key;
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
            if (i + 1 < c) {
                const uint32_t key = order_key(__uint_as_float(e[u].z));
                sh.u.keys[i + 1] = key;
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
        }
        wave_range(sh, kmn, kmx);
        radix_prepare(sh);
        __syncthreads();
        const Kth t = radix_find(sh, LdsKeys{sh.u.keys, c}, k, 32, 0x7FFFFFFF, true);
        emit(sh, LdsSeg{&sh, c, seg}, out, k, t);
        return;
    }
    const Kth t = radix_find(sh, GlobalPairs{cp, c}, k);
    emit(sh, GlobalPairSeg{cp, c, seg}, out, k, t);
}

// Threshold for the sampled pass over a row of n > NLDS scores: 8192 scores
// in 32 evenly spaced runs of 256 give a key tau that somewhat more than k
// entries of the row are expected to reach.  With m = k * 8192 / n samples
// expected at or above the row's k-th largest score, tau is a lower bound of
// the r-th largest sample, r - 4 sqrt(r) = m: the expected pass count r n /
// 8192 then exceeds k by four standard deviations of its sampling error (the
// count of samples above a level is near-binomial, variance about r), so
// fewer than k entries pass only rarely (the caller then takes the exact
// path; the result never depends on tau, only the cost does).
//
// sample_begin issues the loads (16 scores per thread, kept in registers);
// sample_threshold finds tau with the radix select, resolved to at least
// 1/256 of the key range and until at most a quarter more samples than r
// reach it.  Every thread returns tau.
constexpr int RPW = NSB / NW;  // sample runs per wave
struct Samples {
    f32x4 v[RPW];
};

__device__ __forceinline__ Samples sample_begin(const float *row, int64_t n)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    Samples sp;
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const int s = w * RPW + u;
        const int64_t start = ((n - SBL) * s / (NSB - 1)) & ~(int64_t)3;
        sp.v[u] = *reinterpret_cast<const f32x4 *>(row + start + 4 * lane);
    }
    return sp;
}

__device__ uint32_t sample_threshold(Shared &sh, const Samples &sp, int64_t n, int k)
{
    constexpr int IT = 4 * RPW;
    uint32_t key[IT];
    uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        key[4 * u] = order_key(sp.v[u].x);
        key[4 * u + 1] = order_key(sp.v[u].y);
        key[4 * u + 2] = order_key(sp.v[u].z);
        key[4 * u + 3] = order_key(sp.v[u].w);
    }
#pragma unroll
    for (int u = 0; u < IT; ++u) {
        kmn = min(kmn, key[u]);
        kmx = max(kmx, key[u]);
    }
    wave_range(sh, kmn, kmx);
    radix_prepare(sh);
    __syncthreads();
    const float m = (float)k * (float)NSAMP / (float)n;
    const float sr = 0.5f * (4.f + sqrtf(16.f + 4.f * m));
    int r = (int)ceilf(sr * sr);
    r = r < 1 ? 1 : (r > NSAMP ? NSAMP : r);
    // at most a quarter more samples than r at or above tau, and never so
    // many that the expected pass count would crowd the candidate lists
    // (7/8 of their capacity)
    const int64_t cap = (int64_t)NW * CAPW * 7 / 8 * NSAMP / n;
    int64_t mg = r + r / 4 + 4;
    mg = mg < cap ? mg : cap;
    const int max_ge = (int)(mg > r ? mg : r);

    RegKeys<IT> rk;
    rk.valid = (1u << IT) - 1u;
#pragma unroll
    for (int u = 0; u < IT; ++u) rk.k[u] = key[u];
    return radix_find(sh, rk, r, 8, max_ge, true).key;
}

// One streaming pass over row[lo, hi) (lo a multiple of 4): every entry with
// key >= tau goes to its wave's ordered LDS list (wave w takes the w-th
// contiguous part, a multiple of 256 entries long), so the lists visited
// wave by wave are in ascending position order.  sh.wcnt[w] is the count of
// wave w's passing entries (more than CAPW means its list overflowed).
// filter_begin issues the loads of a wave's first 1024 scores (so that they
// can be in flight while tau is found); filter_finish does the pass.
constexpr int FU = 4;  // f32x4 loads per lane per step of the pass
struct FilterPart {
    int64_t lo, hi;  // this wave's part of the range
    f32x4 v[FU];     // its first FU * 256 scores
};

__device__ __forceinline__ FilterPart filter_begin(const float *row, int64_t lo_row, int64_t hi_row)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t seg = (hi_row - lo_row + NW * 256 - 1) / (NW * 256) * 256;
    FilterPart p;
    p.lo = lo_row + (int64_t)w * seg;
    p.hi = min<int64_t>(hi_row, p.lo + seg);
#pragma unroll
    for (int u = 0; u < FU; ++u) {
        const int64_t i = p.lo + u * 256 + 4 * lane;
        p.v[u] = i < p.hi ? *reinterpret_cast<const f32x4 *>(row + i) : f32x4{0, 0, 0, 0};
    }
    return p;
}

__device__ void filter_finish(Shared &sh, const float *row, const FilterPart &p, uint32_t tau)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t lo = p.lo, hi = p.hi;
    int cnt = 0;
    uint32_t *ck = sh.u.cand.key + w * CAPW;
    int32_t *ci = sh.u.cand.idx + w * CAPW;
    f32x4 v[FU];
#pragma unroll
    for (int u = 0; u < FU; ++u) v[u] = p.v[u];
    for (int64_t base = lo; base < hi; base += FU * 256) {
        if (base != lo) {
#pragma unroll
            for (int u = 0; u < FU; ++u) {
                const int64_t i = base + u * 256 + 4 * lane;
                v[u] = i < hi ? *reinterpret_cast<const f32x4 *>(row + i) : f32x4{0, 0, 0, 0};
            }
        }
#pragma unroll
        for (int u = 0; u < FU; ++u) {
            const int64_t i = base + u * 256 + 4 * lane;
            const uint32_t k0 = order_key(v[u].x), k1 = order_key(v[u].y);
            const uint32_t k2 = order_key(v[u].z), k3 = order_key(v[u].w);
            const bool f0 = i < hi && k0 >= tau, f1 = i + 1 < hi && k1 >= tau;
            const bool f2 = i + 2 < hi && k2 >= tau, f3 = i + 3 < hi && k3 >= tau;
            const int c = (int)f0 + (int)f1 + (int)f2 + (int)f3;
            if (ballot(c > 0) == 0) continue;
            const uint64_t b0 = ballot(c & 1), b1 = ballot(c & 2), b2 = ballot(c & 4);
            int q = cnt + lanes_below(b0) + 2 * lanes_below(b1) + 4 * lanes_below(b2);
            if (f0) { if (q < CAPW) { ck[q] = k0; ci[q] = (int32_t)i; } ++q; }
            if (f1) { if (q < CAPW) { ck[q] = k1; ci[q] = (int32_t)(i + 1); } ++q; }
            if (f2) { if (q < CAPW) { ck[q] = k2; ci[q] = (int32_t)(i + 2); } ++q; }
            if (f3) { if (q < CAPW) { ck[q] = k3; ci[q] = (int32_t)(i + 3); } ++q; }
            cnt += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
        }
    }
    if (lane == 0) sh.wcnt[w] = cnt;
    __syncthreads();
}

__device__ __forceinline__ void filter_to_lists(Shared &sh, const float *row, int64_t lo_row, int64_t hi_row,
                                                uint32_t tau)
{
    filter_finish(sh, row, filter_begin(row, lo_row, hi_row), tau);
}

__global__ __launch_bounds__(NT) void select_kernel(SelectArgs a)
{
    __shared__ Shared sh;
    const int tid = threadIdx.x;
    const int t = blockIdx.x, b = blockIdx.y;
    const int64_t n = a.q_pos0 + t + 1;
    const int k = a.top_k;
    const float *row = a.S + ((int64_t)b * a.T_q + t) * a.ld;
    int32_t *out = a.idx + (int64_t)b * a.idx_sb + (int64_t)t * a.idx_st;

    const int m = (int)min<int64_t>(n, k);
    for (int j = m + tid; j < k; j += NT) out[j] = -1;
    if (n <= k) {
        for (int j = tid; j < m; j += NT) out[j] = j;
        return;
    }
    if (a.cand) {
        // after a fused score pass: the row's candidates, unless their count
        // says the row was rescored in full
        const int64_t r = (int64_t)b * a.T_q + t;
        const int c = a.ccnt[r];
        if (!fused_row_bad(c, n, k)) {
            select_from_pairs(sh, a.cand + r * (2 * FUSE_CAP), c, n, out, k);
            return;
        }
    }

    if (n <= NLDS) {
        // ---- path A: whole row in LDS (all loads of a thread issued before
        // the first store; range-checked, so nothing past the row is read)
        constexpr int IT = NLDS / (4 * NT);
        u32x4 v[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) v[u] = ld16_ranged(row, (uint32_t)n * 4u, 16u * (uint32_t)(tid + u * NT));
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        auto put = [&](int i, uint32_t bits) {
            if (i < n) {
                const uint32_t key = order_key(__uint_as_float(bits));
                sh.u.keys[i] = key;
                kmn = min(kmn, key);
                kmx = max(kmx, key);
            }
        };
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int i = 4 * (tid + u * NT);
            put(i, v[u].x);
            put(i + 1, v[u].y);
            put(i + 2, v[u].z);
            put(i + 3, v[u].w);
        }
        wave_range(sh, kmn, kmx);
        radix_prepare(sh);
        __syncthreads();
        const Kth t = radix_find(sh, LdsKeys{sh.u.keys, (int)n}, k, 32, 0x7FFFFFFF, true);
        const int seg = (int)(((n + NW - 1) / NW + 63) / 64 * 64);
        emit(sh, LdsSeg{&sh, (int)n, seg}, out, k, t);
        return;
    }

    // ---- path B: sampled threshold, one streaming pass, exact select on
    // the candidates
    const Samples sp = sample_begin(row, n);          // samples first,
    const FilterPart part = filter_begin(row, 0, n);  // then the pass's first scores (in flight while tau is found)
    const uint32_t tau = sample_threshold(sh, sp, n, k);
    filter_finish(sh, row, part, tau);
    int total = 0;
    bool overflow = false;
    for (int v = 0; v < NW; ++v) {
        total += sh.wcnt[v];
        overflow |= sh.wcnt[v] > CAPW;
    }
    if (!overflow && total >= k) {
        const Kth t = radix_find(sh, Candidates{&sh}, k);
        emit(sh, CandSeg{&sh}, out, k, t);
        return;
    }

    // ---- path C: exact, streaming the row from memory
    __syncthreads();
    const Kth kc = radix_find(sh, GlobalRow{row, n}, k);
    const int64_t seg = ((n + NW - 1) / NW + 63) / 64 * 64;
    emit(sh, GlobalSeg{row, n, seg}, out, k, kc);
}

// The per-segment candidate lists of one row in the workspace, read in
// place: entry i of their concatenation lies in the last segment s with
// pre[s] <= i (pre: list offsets by segment in LDS, INT_MAX past the last
// segment; at most 64 segments), at slot i - pre[s] of segment s's list.
struct SegLists {
    const uint32_t *key;  // the row's first segment list (cap slots per segment)
    const int32_t *idx;
    const int *pre;
    int total, cap;
    __device__ __forceinline__ int64_t src(int i) const
    {
        int s = 0, base = 0;
#pragma unroll
        for (int step = 32; step >= 1; step >>= 1) {
            const int pv = pre[s + step];
            const bool mv = pv <= i;
            s += mv ? step : 0;
            base = mv ? pv : base;
        }
        return (int64_t)s * cap + (i - base);
    }
    template <class F> __device__ void visit(F f) const
    {
        for (int i = threadIdx.x; i < total; i += NT) f(key[src(i)]);
    }
};

struct SegListSeg {
    SegLists l;
    int seg;  // entries per wave run
    __device__ int len(int w) const { return seg; }
    __device__ bool get(int w, int j, uint32_t &key, int32_t &pos) const
    {
        const int i = w * seg + j;
        if (j >= seg || i >= l.total) return false;
        const int64_t e = l.src(i);
        key = l.key[e];
        pos = l.idx[e];
        return true;
    }
};

// ---------------------------------------------------------------------------
// Few long rows: segment filter / final select.
// ---------------------------------------------------------------------------
constexpr int SEG_CAP = 2048;     // candidate slots per segment in the workspace

__device__ __forceinline__ int64_t row_id(const SelectArgs &a, int b, int t) { return (int64_t)b * a.T_q + t; }

// One workgroup per (row, segment): the row's sampled threshold (every
// workgroup of a row finds the same tau from the same samples), then the
// segment's entries at or above it, in position order, into the segment's
// slots of the workspace.
__global__ __launch_bounds__(NT) void select_filter_kernel(SelectArgs a)
{
    __shared__ Shared sh;
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int seg = blockIdx.x, t = blockIdx.y, b = blockIdx.z;
    const int64_t n = a.q_pos0 + t + 1;
    if (n <= a.top_k) return;
    const int64_t r = row_id(a, b, t);
    const int64_t lo = (int64_t)seg * a.seg_len;
    const int64_t hi = min<int64_t>(n, lo + a.seg_len);
    int32_t *cnt = a.cnt + r * a.nseg + seg;
    if (lo >= hi) {
        if (tid == 0) *cnt = 0;
        return;
    }
    const float *row = a.S + r * a.ld;
    const Samples sp = sample_begin(row, n);            // samples first,
    const FilterPart part = filter_begin(row, lo, hi);  // then the segment's first scores (in flight while tau is found)
    const uint32_t tau = sample_threshold(sh, sp, n, a.top_k);
    filter_finish(sh, row, part, tau);
    int off = 0, total = 0;
    bool overflow = false;
    for (int v = 0; v < NW; ++v) {
        if (v < w) off += sh.wcnt[v];
        total += sh.wcnt[v];
        overflow |= sh.wcnt[v] > CAPW;
    }
    if (overflow || total > SEG_CAP) {
        if (tid == 0) *cnt = -1;
        return;
    }
    uint32_t *ok = a.ckey + (r * a.nseg + seg) * SEG_CAP;
    int32_t *oi = a.cidx + (r * a.nseg + seg) * SEG_CAP;
    for (int j = lane; j < sh.wcnt[w]; j += 64) {
        ok[off + j] = sh.u.cand.key[w * CAPW + j];
        oi[off + j] = sh.u.cand.idx[w * CAPW + j];
    }
    if (tid == 0) *cnt = total;
}

// One workgroup per row: the segments' lists gathered into registers
// (ascending positions, segment after segment) and the exact select on them;
// the exact select on the lists in memory when they hold more than the
// registers; the exact path from the row itself when a segment overflowed or
// fewer than k entries passed.
__global__ __launch_bounds__(NT) void select_final_kernel(SelectArgs a)
{
    __shared__ Shared sh;
    __shared__ int pre[128];  // list offsets by segment; past the last segment: INT_MAX
    __shared__ int ptotal;
    const int tid = threadIdx.x;
    const int t = blockIdx.x, b = blockIdx.y;
    const int64_t n = a.q_pos0 + t + 1;
    const int k = a.top_k;
    const int64_t r = row_id(a, b, t);
    const float *row = a.S + r * a.ld;
    int32_t *out = a.idx + (int64_t)b * a.idx_sb + (int64_t)t * a.idx_st;
    const int m = (int)min<int64_t>(n, k);
    for (int j = m + tid; j < k; j += NT) out[j] = -1;
    if (n <= k) {
        for (int j = tid; j < m; j += NT) out[j] = j;
        return;
    }
    if (tid < 64) {
        // segment counts (nseg <= 64) -> exclusive prefix by one wave; a
        // negative count (overflowed segment) marks the row bad (-1 total)
        const int c = tid < a.nseg ? a.cnt[r * a.nseg + tid] : 0;
        const int v = c < 0 ? 0 : c;
        const int inc = wave_prefix_sum(v);
        pre[tid] = tid < a.nseg ? inc - v : 0x7FFFFFFF;
        pre[64 + tid] = 0x7FFFFFFF;
        const bool bad = ballot(c < 0) != 0;
        if (tid == 63) ptotal = bad ? -1 : inc;
    }
    __syncthreads();
    const int total = ptotal;
    if (total >= k && total <= NW * CAPW) {
        // the concatenated lists (ascending positions) cut into NW runs of
        // `run` entries, one per wave, held in registers: thread (w, lane)
        // takes entries w * run + lane + 64 u.  Entry i lies in the last
        // segment s with pre[s] <= i: a branch-free binary search for every
        // entry of a thread first, then all its loads.
        constexpr int IT = NW * CAPW / NT;
        const int w = tid >> 6, lane = tid & 63;
        const int run = ((total + NW - 1) / NW + 63) / 64 * 64;
        int sg[IT], sb[IT];
        RegKeys<IT> rk;
        int32_t pos[IT];
        rk.valid = 0u;
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            sg[u] = 0;
            sb[u] = 0;
            if (64 * u >= run) continue;  // (uniform)
            const int i = w * run + lane + 64 * u;
            if (i < total) rk.valid |= 1u << u;
            int s = 0, base = 0;
#pragma unroll
            for (int step = 32; step >= 1; step >>= 1) {
                const int pv = pre[s + step];
                const bool mv = pv <= i;
                s += mv ? step : 0;
                base = mv ? pv : base;
            }
            sg[u] = s;
            sb[u] = i - base;
        }
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            rk.k[u] = 0u;
            pos[u] = -1;
            if ((rk.valid >> u) & 1u) {
                const int64_t src = (r * a.nseg + sg[u]) * SEG_CAP + sb[u];
                rk.k[u] = a.ckey[src];
                pos[u] = a.cidx[src];
            }
        }
#pragma unroll
        for (int u = 0; u < IT; ++u)
            if ((rk.valid >> u) & 1u) {
                kmn = min(kmn, rk.k[u]);
                kmx = max(kmx, rk.k[u]);
            }
        wave_range(sh, kmn, kmx);
        radix_prepare(sh);
        __syncthreads();
        const Kth t = radix_find(sh, rk, k, 32, 0x7FFFFFFF, true);
        emit_regs(sh, rk, pos, out, k, t);
        return;
    }
    if (total >= k) {
        // more candidates than the registers hold: the exact select on the
        // lists where they lie
        const SegLists l{a.ckey + r * a.nseg * SEG_CAP, a.cidx + r * a.nseg * SEG_CAP, pre, total, SEG_CAP};
        const Kth kl = radix_find(sh, l, k);
        emit(sh, SegListSeg{l, ((total + NW - 1) / NW + 63) / 64 * 64}, out, k, kl);
        return;
    }
    // path C: exact, streaming the row from memory
    const Kth kc = radix_find(sh, GlobalRow{row, n}, k);
    const int64_t seg = ((n + NW - 1) / NW + 63) / 64 * 64;
    emit(sh, GlobalSeg{row, n, seg}, out, k, kc);
}

struct MultiPlan {
    bool on;
    int nseg;
    int64_t seg_len;
};

MultiPlan multi_plan(int B, int T_q, int64_t q_pos0)
{
    const int64_t rows = (int64_t)B * T_q, n_max = q_pos0 + T_q;
    if (rows > 128 || n_max < 32768) return {false, 1, 0};
    int64_t nseg = (512 + rows - 1) / rows;
    if (nseg > 64) nseg = 64;
    int64_t seg = (n_max + nseg - 1) / nseg;
    seg = (seg + NW * 256 - 1) / (NW * 256) * (NW * 256);
    nseg = (n_max + seg - 1) / seg;
    return {true, (int)nseg, seg};
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

}  // namespace

size_t select_ws_bytes(int B, int T_q, int64_t q_pos0)
{
    const MultiPlan p = multi_plan(B, T_q, q_pos0);
    if (!p.on) return 0;
    const size_t rows = (size_t)B * T_q;
    return align256(rows * p.nseg * 4) + 2 * align256(rows * p.nseg * SEG_CAP * 4);
}

hipError_t launch_select(const SelectArgs &a_in, void *extra, hipStream_t st)
{
    const MultiPlan p = multi_plan(a_in.B, a_in.T_q, a_in.q_pos0);
    if (!p.on || a_in.cand) {
        hipLaunchKernelGGL(select_kernel, dim3(a_in.T_q, a_in.B), dim3(NT), 0, st, a_in);
        return hipGetLastError();
    }
    SelectArgs a = a_in;
    const size_t rows = (size_t)a.B * a.T_q;
    uint8_t *ws = (uint8_t *)extra;
    a.nseg = p.nseg;
    a.seg_len = p.seg_len;
    a.cnt = (int32_t *)ws;
    ws += align256(rows * p.nseg * 4);
    a.ckey = (uint32_t *)ws;
    ws += align256(rows * p.nseg * SEG_CAP * 4);
    a.cidx = (int32_t *)ws;
    hipLaunchKernelGGL(select_filter_kernel, dim3(a.nseg, a.T_q, a.B), dim3(NT), 0, st, a);
    hipLaunchKernelGGL(select_final_kernel, dim3(a.T_q, a.B), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcsi
