// Measurement helpers (not steps of the method): the practical ceiling of
// the indexer score kernel's matrix-core work on this chip, of a plain
// streaming read from HBM (the roof of the memory-bound decode kernels), and
// of a gather of whole rows into LDS (the sparse attention's memory
// pattern without its arithmetic).  A loop issues
// the score kernel's instruction stream -- per 32-key block and wave, 16
// v_mfma_f32_32x32x16_bf16 in two accumulator chains (two 32-row tiles of
// (query, head) rows against the block's keys, 8 k-steps of 16 dims) -- at
// the same occupancy (8 waves per workgroup, two per SIMD) and d map (the
// two lanes of a key hold adjacent 8-dim chunks: d = 16*s + 8*g + e), on operands
// drawn like the indexer's (the caller passes N(0,1)/8 bf16 values), but
// with nothing else: no ReLU / weight / head-reduction epilogue, no score
// stores, no key traffic from memory.
//   mode 0: B fragments in registers, four blocks' worth, rotated block by
//           block (the operands change every block, as they do when keys
//           stream through).
//   mode 1: B fragments read from two key tiles staged once in LDS (128
//           keys x 128 dims, rows padded by 16 bytes), block by block, with
//           the score kernel's reads.
// Each wave finally stores one float (the sum of its accumulators), so no
// product is dead.  Work per launch: n_wg * 8 waves * blocks * 16 * 32768
// flop.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lcsi_ceiling.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int NWAVE = 8;
constexpr int KS = 8;              // k-steps of 16 dims (128 dims)
constexpr int ROWB = 128 * 2 + 16; // LDS bytes per key row (+16 B pad), as in the score kernel
constexpr int KT = 128;            // keys per LDS tile

__device__ __forceinline__ bf16x8 ld_frag(const uint16_t *p) { return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(p)); }

template <int MODE>
__global__ __launch_bounds__(NWAVE * 64) __attribute__((amdgpu_waves_per_eu(2))) void mfma_loop_kernel(
    const uint16_t *data, float *out, int blocks)
{
    // (mode 1 asks for 96 KB of LDS so that, like the score kernel, one
    // workgroup -- two waves per SIMD -- runs per CU)
    __shared__ __attribute__((aligned(1024))) uint8_t tiles[MODE == 1 ? 96 * 1024 : 16];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, l32 = lane & 31, g = lane >> 5;
    // A fragments: rows (lane % 32) of two 32-row tiles, 8 dims of group g per k-step
    const uint16_t *qb = data + ((size_t)(blockIdx.x % 64) * NWAVE + wave) * 64 * 128;
    bf16x8 qa[2][KS];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < KS; ++s) qa[rt][s] = ld_frag(qb + (rt * 32 + l32) * 128 + 16 * s + 8 * g);
    const uint16_t *kbase = data + (size_t)64 * NWAVE * 64 * 128;  // keys after the query rows
    f32x16 acc0 = f32x16{0}, acc1 = f32x16{0};
    if constexpr (MODE == 0) {
        bf16x8 bk[4][KS];
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int s = 0; s < KS; ++s) bk[j][s] = ld_frag(kbase + (j * 32 + l32) * 128 + 16 * s + 8 * g);
        for (int it = 0; it < blocks; it += 4) {
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bk[j][s], acc0, 0, 0, 0);
                    acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bk[j][s], acc1, 0, 0, 0);
                }
        }
    } else {
        // two tiles of 128 keys staged once (rows padded as in the score kernel)
        for (int c = tid; c < 2 * KT * 16; c += NWAVE * 64) {
            const int row = c / 16, part = c % 16;
            *reinterpret_cast<u32x4 *>(tiles + row * ROWB + part * 16) =
                *reinterpret_cast<const u32x4 *>(kbase + (size_t)row * 128 + part * 8);
        }
        __syncthreads();
        for (int it = 0; it < blocks; ++it) {
            const int cb = it & 7;  // block cb of the 8 blocks in the two tiles
            const uint8_t *src = tiles + (cb * 32 + l32) * ROWB + g * 16;
            bf16x8 bk[KS];
#pragma unroll
            for (int s = 0; s < KS; ++s) bk[s] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(src + 32 * s));
#pragma unroll
            for (int s = 0; s < KS; ++s) {
                acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[0][s], bk[s], acc0, 0, 0, 0);
                acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[1][s], bk[s], acc1, 0, 0, 0);
            }
        }
    }
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += acc0[i] + acc1[i];
    for (int o = 32; o >= 1; o >>= 1) sum += __shfl_xor(sum, o);
    if (lane == 0) out[(size_t)blockIdx.x * NWAVE + wave] = sum;
}

// Streaming read: every 16-byte unit of the buffer once (grid-stride, eight
// loads in flight per thread, non-temporal), XOR-reduced to one word per
// thread so no load is dead.
__global__ __launch_bounds__(256) void read_kernel(const u32x4 *p, size_t n16, uint32_t *out)
{
    constexpr int U = 8;
    const size_t tid = (size_t)blockIdx.x * blockDim.x + threadIdx.x, stride = (size_t)gridDim.x * blockDim.x;
    u32x4 acc{0, 0, 0, 0};
    size_t i = tid;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= v[u];
    }
    for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(p + i);
    out[tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

// Gather: workgroup w takes its `tiles` lists of 32 row numbers (idx + w *
// tiles * 32, clamped to [0, n_rows)) and copies each list's rows straight
// from memory into one of two LDS buffers with direct 16-byte loads (lane l
// of load m fills 16-byte slot 64m + l = chunk c of list entry r, as the
// attention kernel does), the next list in flight while the last one is read
// back: each thread XORs one 16-byte LDS unit per list into its output word.
constexpr int GW = 4;                                // waves per workgroup
constexpr int GMAX_ROWB = 1152;                      // largest row
constexpr int GMAX_TILES = 64;                       // largest list count
constexpr int GBUF = 32 * GMAX_ROWB;                 // bytes per buffer

__device__ __forceinline__ void lds_dma16(const void *src, uint8_t *lds)
{
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
#else
    (void)src;
    (void)lds;
#endif
}

__global__ __launch_bounds__(GW * 64) void gather_kernel(const uint8_t *rows, int64_t n_rows, uint32_t row_bytes,
                                                         const int32_t *idx, int tiles, uint32_t *out)
{
    __shared__ __attribute__((aligned(1024))) uint8_t gb0[GBUF];
    __shared__ __attribute__((aligned(1024))) uint8_t gb1[GBUF];
    __shared__ int32_t sidx[GMAX_TILES * 32];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int cpr = (int)(row_bytes / 16);  // 16-byte chunks per row
    const int nload = (32 * cpr + 63) / 64;  // direct loads per list
    const int32_t *il = idx + (int64_t)blockIdx.x * tiles * 32;
    for (int i = tid; i < tiles * 32; i += GW * 64) {
        const int32_t v = il[i];
        sidx[i] = v < 0 ? 0 : (v >= n_rows ? (int32_t)(n_rows - 1) : v);
    }
    __syncthreads();
    auto issue = [&](int t, uint8_t *dst) {
        for (int m = wave; m < nload; m += GW) {
            const int slot = 64 * m + lane, r = slot / cpr, c = slot - r * cpr;
            if (r < 32) lds_dma16(rows + (uint64_t)sidx[t * 32 + r] * row_bytes + 16 * c, dst + 1024 * m);
        }
    };
    u32x4 acc{0, 0, 0, 0};
    auto step = [&](int t, const uint8_t *cur, uint8_t *next) {
        if (t + 1 < tiles) issue(t + 1, next);
        acc ^= *reinterpret_cast<const u32x4 *>(cur + 16 * tid);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
    };
    issue(0, gb0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    for (int t = 0; t < tiles; t += 2) {
        step(t, gb0, gb1);
        if (t + 1 >= tiles) break;
        step(t + 1, gb1, gb0);
    }
    out[(size_t)blockIdx.x * GW * 64 + tid] = acc.x ^ acc.y ^ acc.z ^ acc.w;
}

}  // namespace

extern "C" {

int lcsi_ceiling_gather(const void *rows, int64_t n_rows, uint32_t row_bytes, const int32_t *idx, int n_wg,
                        int tiles, uint32_t *out, void *stream)
{
    if (!rows || !idx || !out || n_rows < 1 || n_wg < 1 || tiles < 1 || tiles > GMAX_TILES || row_bytes < 16 ||
        row_bytes > GMAX_ROWB || row_bytes % 16)
        return -1;
    if (((uintptr_t)rows % 16) || ((uintptr_t)idx % 4) || ((uintptr_t)out % 4)) return -5;
    hipLaunchKernelGGL(gather_kernel, dim3(n_wg), dim3(GW * 64), 0, (hipStream_t)stream,
                       reinterpret_cast<const uint8_t *>(rows), n_rows, row_bytes, idx, tiles, out);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

int lcsi_ceiling_read(const void *data, size_t bytes, uint32_t *out, int n_wg, void *stream)
{
    if (!data || !out || n_wg < 1 || bytes < 16 || bytes % 16) return -1;
    if (((uintptr_t)data % 16) || ((uintptr_t)out % 4)) return -5;
    hipLaunchKernelGGL(read_kernel, dim3(n_wg), dim3(256), 0, (hipStream_t)stream,
                       reinterpret_cast<const u32x4 *>(data), bytes / 16, out);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

size_t lcsi_ceiling_data_elems(void) { return (size_t)64 * NWAVE * 64 * 128 + 2 * KT * 128; }

int lcsi_ceiling_mfma(const uint16_t *data, float *out, int n_wg, int blocks, int mode, void *stream)
{
    if (!data || !out || n_wg < 1 || blocks < 4 || blocks % 4 || (mode != 0 && mode != 1)) return -1;
    if (((uintptr_t)data % 16) || ((uintptr_t)out % 4)) return -5;
    hipStream_t s = (hipStream_t)stream;
    if (mode == 0)
        hipLaunchKernelGGL(mfma_loop_kernel<0>, dim3(n_wg), dim3(NWAVE * 64), 0, s, data, out, blocks);
    else
        hipLaunchKernelGGL(mfma_loop_kernel<1>, dim3(n_wg), dim3(NWAVE * 64), 0, s, data, out, blocks);
    return hipGetLastError() == hipSuccess ? 0 : -6;
}

}  // extern "C"
