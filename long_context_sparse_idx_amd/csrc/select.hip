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
//     a threshold tau expected to pass ~2.5k entries; one streaming pass
//     keeps every entry with key >= tau in per-wave ordered LDS lists, and
//     the exact select runs on those.  If fewer than k entries pass, or a
//     list overflows, the row falls back to C.  The result never depends on
//     the sample, only the cost does.
//  C  exact radix select and compaction streaming the row from memory.
//
// Few long rows (decode: a handful of sequences, each with up to a million
// scores) would leave most of the chip idle with one workgroup per row, so
// they take a three-kernel form of path B: one workgroup per row finds the
// sampled threshold; many workgroups per row filter one segment each into
// a per-segment candidate list in the workspace (ordered); one workgroup
// per row gathers the lists (ascending positions, segment after segment)
// and runs the exact select on them -- or path C when a segment overflowed
// or fewer than k entries passed.
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
        uint32_t samp[NSAMP];                    // path B, before filtering
        struct {
            uint32_t key[NW * CAPW];
            int32_t idx[NW * CAPW];
        } cand;                                  // path B candidates
    } u;
    uint32_t hist[NSUB][256];
    int wcnt[NW];
    int wgt[NW];
    int wtie[NW];
    uint32_t kth;
    int rem;
    int ge;
    int full;  // the bin holding the rank-th key is taken whole
    uint32_t wmin[NW], wmax[NW];  // per-wave key range, written while filling LDS
    uint32_t kmin, kmax;
};

// ---- element visitors: each thread calls f(key) for its share ------------

struct LdsKeys {
    const uint32_t *keys;
    int n;
    template <class F> __device__ void visit(F f) const
    {
        for (int i = threadIdx.x; i < n; i += NT) f(keys[i]);
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
// keys).  On return sh.kth is that key and sh.rem the number of entries
// equal to it that belong to the top `rank`.
//
// A first pass finds the smallest and largest key; the 8-bit digit passes
// then run on the offset key - kmin, starting at the highest bit of the
// range kmax - kmin, so the first 256 bins span the keys actually present
// (scores of one row share sign and exponent bits, and a digit over those
// bits would put nearly every key into one or two bins).
// resolve < 32 stops once that many offset bits from the top are fixed and
// at most max_ge keys lie at or above the current bin: sh.kth is then kmin +
// the offset prefix with the lower bits cleared -- a lower bound of the
// rank-th key that at least `rank` and at most max_ge keys reach (used for
// the sampled threshold, where only a bound is needed; max_ge keeps the
// bound tight when the keys span a wide range, e.g. scores of both signs).
// The smallest and largest of a thread's keys (kmn, kmx) reduced over the
// wave into its slot of sh.wmin / sh.wmax (every wave writes its slot; a
// wave without keys writes the empty range).  Callers that fill LDS do this
// before the barrier that ends the fill, so radix_find(..., ranged = true)
// needs no pass of its own over the keys for their range.
__device__ __forceinline__ void wave_range(Shared &sh, uint32_t kmn, uint32_t kmx)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        kmn = min(kmn, (uint32_t)__shfl_xor(kmn, o));
        kmx = max(kmx, (uint32_t)__shfl_xor(kmx, o));
    }
    if ((threadIdx.x & 63) == 0) {
        sh.wmin[threadIdx.x >> 6] = kmn;
        sh.wmax[threadIdx.x >> 6] = kmx;
    }
}

template <class Src>
__device__ void radix_find(Shared &sh, const Src &src, int rank, int resolve = 32, int max_ge = 0x7FFFFFFF,
                           bool ranged = false)
{
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    uint32_t kmin_all = 0xFFFFFFFFu, kmax_all = 0u;
    if (ranged) {
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            kmin_all = min(kmin_all, sh.wmin[v]);
            kmax_all = max(kmax_all, sh.wmax[v]);
        }
    } else {
        if (tid == 0) {
            sh.kmin = 0xFFFFFFFFu;
            sh.kmax = 0u;
        }
        __syncthreads();
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
        src.visit([&](uint32_t key) {
            kmn = min(kmn, key);
            kmx = max(kmx, key);
        });
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            kmn = min(kmn, (uint32_t)__shfl_xor(kmn, o));
            kmx = max(kmx, (uint32_t)__shfl_xor(kmx, o));
        }
        if (lane == 0) {
            atomicMin(&sh.kmin, kmn);
            atomicMax(&sh.kmax, kmx);
        }
        __syncthreads();
        kmin_all = sh.kmin;
        kmax_all = sh.kmax;
    }
    const uint32_t kmin = kmin_all, range = kmax_all - kmin;
    if (range == 0) {  // all keys equal: the rank-th is that key
        if (tid == 0) {
            sh.kth = kmin;
            sh.rem = rank;
        }
        __syncthreads();
        return;
    }
    const int msb = 31 - __builtin_clz(range);
    uint32_t mask = msb == 31 ? 0u : ~((2u << msb) - 1u);  // offset bits already fixed (all zero)
    uint32_t prefix = 0;                                    // fixed offset bits
    int rem = rank;
    int hi = msb;  // highest bit of the next digit
#pragma unroll 1
    while (true) {
        const int shift = hi >= 7 ? hi - 7 : 0;
        const uint32_t dmask = (2u << (hi - shift)) - 1u;  // digit width hi-shift+1 <= 8 bits
        for (int i = tid; i < NSUB * 256; i += NT) (&sh.hist[0][0])[i] = 0;
        __syncthreads();
        uint32_t *hw = sh.hist[w % NSUB];
        src.visit([&](uint32_t key) {
            const uint32_t off = key - kmin;
            if ((off & mask) == prefix) atomicAdd(&hw[(off >> shift) & dmask], 1u);
        });
        __syncthreads();
        if (tid < 64) {
            uint32_t c[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                uint32_t v = 0;
#pragma unroll
                for (int h = 0; h < NSUB; ++h) v += sh.hist[h][4 * lane + e];
                c[e] = v;
            }
            const int tot = (int)(c[0] + c[1] + c[2] + c[3]);
            int suf = tot;  // inclusive suffix sum over lanes >= this one
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const int t = __shfl_down(suf, o);
                if (lane + o < 64) suf += t;
            }
            const int above = suf - tot;
            if (above < rem && rem <= suf) {
                int acc = above;
                for (int e = 3; e >= 0; --e) {
                    if (acc + (int)c[e] >= rem) {
                        sh.kth = prefix | ((uint32_t)(4 * lane + e) << shift);
                        sh.rem = rem - acc;
                        sh.ge = (rank - rem) + acc + (int)c[e];  // keys at or above this bin
                        sh.full = (int)c[e] == rem - acc;
                        break;
                    }
                    acc += (int)c[e];
                }
            }
        }
        __syncthreads();
        prefix = sh.kth;
        rem = sh.rem;
        mask |= dmask << shift;
        if (shift == 0 || (msb - shift + 1 >= resolve && sh.ge <= max_ge)) break;
        if (resolve == 32 && sh.full && prefix != 0) {
            // every key of the bin is taken: the keys above offset prefix - 1
            // (this bin and everything above it) are exactly the top `rank`,
            // so the threshold is prefix - 1 with no ties to count
            prefix -= 1;
            rem = 0;
            break;
        }
        hi = shift - 1;
    }
    __syncthreads();  // every thread has read sh.kth / sh.rem above
    if (tid == 0) {
        sh.kth = kmin + prefix;
        sh.rem = rem;
    }
    __syncthreads();
}

// Ordered compaction over per-wave segments visited in ascending position
// order.  Seg::get(w, j, key, pos) returns false past the end of segment w;
// Seg::len(w) is an upper bound on its length (a multiple of 64 not needed).
template <class Seg>
__device__ void emit(Shared &sh, const Seg &seg, int32_t *out, int k)
{
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const uint32_t kth = sh.kth;
    const int need = sh.rem;
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
    gt = wave_sum_int(gt);
    tie = wave_sum_int(tie);
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
        __syncthreads();
        radix_find(sh, LdsKeys{sh.u.cand.key, c}, k, 32, 0x7FFFFFFF, true);
        emit(sh, LdsPairSeg{&sh, c, seg}, out, k);
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
        __syncthreads();
        radix_find(sh, LdsKeys{sh.u.keys, c}, k, 32, 0x7FFFFFFF, true);
        emit(sh, LdsSeg{&sh, c, seg}, out, k);
        return;
    }
    radix_find(sh, GlobalPairs{cp, c}, k);
    emit(sh, GlobalPairSeg{cp, c, seg}, out, k);
}

// Threshold for the sampled pass over a row of n > NLDS scores: 8192 scores
// in 32 evenly spaced runs of 256 give the key tau that about 2.5k entries
// of the row are expected to reach.  Every thread returns tau.
__device__ uint32_t sampled_threshold(Shared &sh, const float *row, int64_t n, int k)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    constexpr int RPW = NSB / NW;  // runs per wave, all loads issued first
    f32x4 v[RPW];
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        const int s = w * RPW + u;
        const int64_t start = ((n - SBL) * s / (NSB - 1)) & ~(int64_t)3;
        v[u] = *reinterpret_cast<const f32x4 *>(row + start + 4 * lane);
    }
#pragma unroll
    for (int u = 0; u < RPW; ++u) {
        uint32_t *d = sh.u.samp + (w * RPW + u) * SBL + 4 * lane;
        d[0] = order_key(v[u].x);
        d[1] = order_key(v[u].y);
        d[2] = order_key(v[u].z);
        d[3] = order_key(v[u].w);
    }
    __syncthreads();
    int64_t r = (5 * (int64_t)k * NSAMP + 2 * n - 1) / (2 * n);
    r = r < 1 ? 1 : (r > NSAMP ? NSAMP : r);
    // a lower bound of the r-th sampled key, resolved to 1/256 of the
    // samples' key range, is precise enough for a threshold -- unless its
    // bin holds so many samples that the expected pass count would crowd
    // the candidate lists (7/8 of their capacity); then refine further
    const int64_t cap = (int64_t)NW * CAPW * 7 / 8 * NSAMP / n;
    radix_find(sh, LdsKeys{sh.u.samp, NSAMP}, (int)r, 8, (int)(cap > r ? cap : r));
    const uint32_t tau = sh.kth;
    __syncthreads();  // every thread has read tau before the lists overwrite the samples
    return tau;
}

// One streaming pass over row[lo, hi) (lo a multiple of 4): every entry with
// key >= tau goes to its wave's ordered LDS list (wave w takes the w-th
// contiguous part, a multiple of 256 entries long), so the lists visited
// wave by wave are in ascending position order.  sh.wcnt[w] is the count of
// wave w's passing entries (more than CAPW means its list overflowed).
__device__ void filter_to_lists(Shared &sh, const float *row, int64_t lo_row, int64_t hi_row, uint32_t tau)
{
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t seg = (hi_row - lo_row + NW * 256 - 1) / (NW * 256) * 256;
    const int64_t lo = lo_row + (int64_t)w * seg;
    const int64_t hi = min<int64_t>(hi_row, lo + seg);
    int cnt = 0;
    uint32_t *ck = sh.u.cand.key + w * CAPW;
    int32_t *ci = sh.u.cand.idx + w * CAPW;
    constexpr int U = 4;
    for (int64_t base = lo; base < hi; base += U * 256) {
        f32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + 4 * lane;
            v[u] = i < hi ? *reinterpret_cast<const f32x4 *>(row + i) : f32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t i = base + u * 256 + 4 * lane;
            const uint32_t k0 = order_key(v[u].x), k1 = order_key(v[u].y);
            const uint32_t k2 = order_key(v[u].z), k3 = order_key(v[u].w);
            const bool f0 = i < hi && k0 >= tau, f1 = i + 1 < hi && k1 >= tau;
            const bool f2 = i + 2 < hi && k2 >= tau, f3 = i + 3 < hi && k3 >= tau;
            const int c = (int)f0 + (int)f1 + (int)f2 + (int)f3;
            if (ballot(c > 0) == 0) continue;
            const uint64_t b0 = ballot(c & 1), b1 = ballot(c & 2), b2 = ballot(c & 4);
            int p = cnt + lanes_below(b0) + 2 * lanes_below(b1) + 4 * lanes_below(b2);
            if (f0) { if (p < CAPW) { ck[p] = k0; ci[p] = (int32_t)i; } ++p; }
            if (f1) { if (p < CAPW) { ck[p] = k1; ci[p] = (int32_t)(i + 1); } ++p; }
            if (f2) { if (p < CAPW) { ck[p] = k2; ci[p] = (int32_t)(i + 2); } ++p; }
            if (f3) { if (p < CAPW) { ck[p] = k3; ci[p] = (int32_t)(i + 3); } ++p; }
            cnt += __popcll(b0) + 2 * __popcll(b1) + 4 * __popcll(b2);
        }
    }
    if (lane == 0) sh.wcnt[w] = cnt;
    __syncthreads();
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
        __syncthreads();
        radix_find(sh, LdsKeys{sh.u.keys, (int)n}, k, 32, 0x7FFFFFFF, true);
        const int seg = (int)(((n + NW - 1) / NW + 63) / 64 * 64);
        emit(sh, LdsSeg{&sh, (int)n, seg}, out, k);
        return;
    }

    // ---- path B: sampled threshold, one streaming pass, exact select on
    // the candidates
    const uint32_t tau = sampled_threshold(sh, row, n, k);
    filter_to_lists(sh, row, 0, n, tau);
    int total = 0;
    bool overflow = false;
    for (int v = 0; v < NW; ++v) {
        total += sh.wcnt[v];
        overflow |= sh.wcnt[v] > CAPW;
    }
    if (!overflow && total >= k) {
        radix_find(sh, Candidates{&sh}, k);
        emit(sh, CandSeg{&sh}, out, k);
        return;
    }

    // ---- path C: exact, streaming the row from memory
    __syncthreads();
    radix_find(sh, GlobalRow{row, n}, k);
    const int64_t seg = ((n + NW - 1) / NW + 63) / 64 * 64;
    emit(sh, GlobalSeg{row, n, seg}, out, k);
}

// ---------------------------------------------------------------------------
// Few long rows: threshold / segment filter / final select.
// ---------------------------------------------------------------------------
constexpr int SEG_CAP = 2048;     // candidate slots per segment in the workspace

__device__ __forceinline__ int64_t row_id(const SelectArgs &a, int b, int t) { return (int64_t)b * a.T_q + t; }

__global__ __launch_bounds__(NT) void select_thresh_kernel(SelectArgs a)
{
    __shared__ Shared sh;
    const int t = blockIdx.x, b = blockIdx.y;
    const int64_t n = a.q_pos0 + t + 1;
    if (n <= a.top_k) return;
    const float *row = a.S + row_id(a, b, t) * a.ld;
    const uint32_t tau = sampled_threshold(sh, row, n, a.top_k);
    if (threadIdx.x == 0) a.tau[row_id(a, b, t)] = tau;
}

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
    filter_to_lists(sh, a.S + r * a.ld, lo, hi, a.tau[r]);
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

__global__ __launch_bounds__(NT) void select_final_kernel(SelectArgs a)
{
    __shared__ Shared sh;
    __shared__ int pre[65];
    const int tid = threadIdx.x, w = tid >> 6;
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
        int inc = v;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
            const int u = __shfl_up(inc, o);
            if (tid >= o) inc += u;
        }
        if (tid < a.nseg) pre[tid] = inc - v;
        const bool bad = ballot(c < 0) != 0;
        if (tid == a.nseg - 1) pre[a.nseg] = bad ? -1 : inc;
    }
    __syncthreads();
    const int total = pre[a.nseg];
    if (total >= k && total <= NW * CAPW) {
        // the concatenated lists, contiguous in LDS (ascending positions);
        // every load of a thread is issued before the first store
        constexpr int IT = NW * CAPW / NT;
        uint32_t kv[IT];
        int32_t iv[IT];
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int i = tid + u * NT;
            kv[u] = 0u;
            iv[u] = 0;
            if (i < total) {
                // segment holding entry i: the last s with pre[s] <= i
                // (binary search over the ascending prefix; pre[0] = 0)
                int s = 0;
                for (int step = 32; step >= 1; step >>= 1)
                    if (s + step < a.nseg && pre[s + step] <= i) s += step;
                const int64_t src = (r * a.nseg + s) * SEG_CAP + (i - pre[s]);
                kv[u] = a.ckey[src];
                iv[u] = a.cidx[src];
            }
        }
        uint32_t kmn = 0xFFFFFFFFu, kmx = 0u;
#pragma unroll
        for (int u = 0; u < IT; ++u) {
            const int i = tid + u * NT;
            if (i < total) {
                sh.u.cand.key[i] = kv[u];
                sh.u.cand.idx[i] = iv[u];
                kmn = min(kmn, kv[u]);
                kmx = max(kmx, kv[u]);
            }
        }
        wave_range(sh, kmn, kmx);
        __syncthreads();
        radix_find(sh, LdsKeys{sh.u.cand.key, total}, k, 32, 0x7FFFFFFF, true);
        const int seg = ((total + NW - 1) / NW + 63) / 64 * 64;
        emit(sh, LdsPairSeg{&sh, total, seg}, out, k);
        return;
    }
    // path C: exact, streaming the row from memory
    (void)w;
    radix_find(sh, GlobalRow{row, n}, k);
    const int64_t seg = ((n + NW - 1) / NW + 63) / 64 * 64;
    emit(sh, GlobalSeg{row, n, seg}, out, k);
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
    return align256(rows * 4) + align256(rows * p.nseg * 4) + 2 * align256(rows * p.nseg * SEG_CAP * 4);
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
    a.tau = (uint32_t *)ws;
    ws += align256(rows * 4);
    a.cnt = (int32_t *)ws;
    ws += align256(rows * p.nseg * 4);
    a.ckey = (uint32_t *)ws;
    ws += align256(rows * p.nseg * SEG_CAP * 4);
    a.cidx = (int32_t *)ws;
    hipLaunchKernelGGL(select_thresh_kernel, dim3(a.T_q, a.B), dim3(NT), 0, st, a);
    hipLaunchKernelGGL(select_filter_kernel, dim3(a.nseg, a.T_q, a.B), dim3(NT), 0, st, a);
    hipLaunchKernelGGL(select_final_kernel, dim3(a.T_q, a.B), dim3(NT), 0, st, a);
    return hipGetLastError();
}

}  // namespace lcsi
