// Prefill GEMM: Y = X W^T for many tokens (M > 16) from a GEMM plan.
//
// "Variable Bit-width Quantization" (mlsanity.com page, Abstract) stores every
// 64-weight group with its own width from {1, 2, 4, 8} and decodes with fused
// dequantize-and-multiply kernels.  With many tokens the product is a dense
// contraction over K, so this path runs it on the matrix cores: each tile of
// the weights is dequantized once into LDS as fp16 and multiplied against the
// tokens with v_mfma_f32_32x32x16_f16 (fp32 accumulation).
//
// GEMM plan (prepared once per matrix, see include/vbq.h): tiles of 128 rows
// x 128 columns (two groups); in a tile the groups are bucketed by width so
// that a wavefront dequantizes 64 groups of one width at a time.
//
// Kernel (512 threads, one workgroup per 128-row block x 32*MT tokens x one
// K-split; the buffers fill the LDS, so one workgroup per compute unit and two
// wavefronts per SIMD, which hide each other's LDS and matrix-core latencies):
//   - a ring of 3 LDS slots receives the raw tiles by LDS-DMA, two tiles
//     ahead of the one being dequantized (wavefronts 0..3 copy);
//   - the tile of chunk k+1 is dequantized into the free half of a double
//     buffer W[2][128 rows][128 k-slots] while the MFMAs consume chunk k
//     (every wavefront takes its share of both);
//   - the tokens' activations of chunk k+1 are copied by LDS-DMA into
//     X[2][32*MT][128 k-slots] from a copy of X in the same k-slot order
//     that a first kernel writes into the workspace.
// Every global read of the loop is an LDS-DMA copy with explicit vmcnt waits,
// so that the tile copies stay in flight across iterations.
// K-slot order inside a group: slot 2j holds column j and slot 2j+1 column
// j + 32 (j < 32), the order in which a group's code word d carries its codes
// (half 0 in the low 16 bits, half 1 in the high 16 bits), so one unpacked
// 32-bit word is one pair of fp16 weights.  The contraction does not depend
// on the order of k as long as W and X use the same one.
#include "vbq_host.h"
#include "vbq_common.h"

#include <algorithm>

using namespace vbq;

namespace {

constexpr int kBN = 128;     // weight rows per tile
constexpr int kTG = 2;       // groups per tile (128 columns)
constexpr int kGT = 256;     // threads per workgroup of the preparation kernels
constexpr int kGW = kGT / 64; // their wavefronts; also the GEMM kernel's LDS-DMA wavefronts
constexpr int kMT = 512;     // threads per workgroup of the GEMM kernel: two wavefronts per SIMD
constexpr int kMW = kMT / 64;
static_assert(kBN * kTG == kGT, "the preparation kernels take one cell of a tile per thread");
constexpr int kGHdr = 16;    // tile header bytes
constexpr int kRing = 3;     // tiles in the LDS ring
constexpr int kLdw = 136;    // LDS row stride of the W and X chunks, in halves (128 + 8 against bank conflicts)
constexpr uint32_t kWBytes = kBN * kLdw * 2; // one W chunk
constexpr uint32_t kGLds = 160u * 1024u;
constexpr int kMaxK = 32768; // 256 chunks: the kernel keeps a split's tile offsets in 4 registers per lane
constexpr int kMaxGemmM = 1 << 20;

typedef _Float16 hf2 __attribute__((ext_vector_type(2)));
typedef _Float16 hf8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// LDS byte address of a pointer into __shared__ memory.
__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (m0 = lds_base, wave-uniform).  Written as asm so the compiler does not tie
// later LDS reads to it with a vmcnt wait: completion is awaited explicitly
// (wait_vm / wait_vm0) before the barrier that publishes the data.  The s_nop
// separates the compiler's m0 write from the LDS-DMA load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// s_waitcnt vmcnt(n) for a run-time n (clamped: a smaller n only waits longer).
__device__ __forceinline__ void wait_vm(int n)
{
    switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
    }
}

__device__ __forceinline__ uint32_t h2u(hf2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ hf2 u2h(uint32_t v) { return __builtin_bit_cast(hf2, v); }

// ---------------------------------------------------------------------------
// Plan preparation.

struct GPrep {
    const uint8_t *blob;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    int N, G, nS, kc;
    uint8_t *buf;       // plan buffer (fill), null for sizing
    uint32_t *table;    // buf's offset table (size pass with a buffer, scan, fill)
    uint32_t *stats;    // sizing without a buffer: [0] largest tile, [2..3] u64 sum of tiles in 16-byte units
    uint32_t *status;   // fill: VBQ_STATUS_PLAN when the blob does not fit the plan (may be null)
    uint32_t max_tile;  // fill: the largest tile the plan was sized for
};

// The cell of thread u of a tile's workgroup: column gl = u / 128 of the
// tile, row r = u % 128 (the slot order inside a width bucket); its width
// code, or -1 outside the matrix.
struct Cell {
    int r, gl, n, g, c;
};

__device__ __forceinline__ Cell tile_cell(const GPrep &a, int nbi, int kci, int u)
{
    Cell e;
    e.r = u & (kBN - 1);
    e.gl = u >> 7;
    e.n = nbi * kBN + e.r;
    e.g = kci * kTG + e.gl;
    e.c = -1;
    if (e.n < a.N && e.g < a.G) {
        const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
        const uint64_t rs = (uint64_t)e.n * a.nS + (e.g >> 5);
        e.c = width_code(wmap[2 * rs], wmap[2 * rs + 1], e.g & 31);
    }
    return e;
}

// Per-width cell counts of the tile (cnt[c], c = log2 b) and this thread's rank
// among the tile's cells of its width (thread order).  wc: LDS [kGW][4].
__device__ __forceinline__ uint32_t width_counts(int c, uint32_t (*wc)[4], uint32_t cnt[4])
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t rank = 0;
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
        const unsigned long long m = __ballot(c == cc);
        if (lane == 0)
            wc[wave][cc] = (uint32_t)__popcll(m);
        if (c == cc)
            rank = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    }
    __syncthreads();
#pragma unroll
    for (int cc = 0; cc < 4; cc++) {
        uint32_t t = 0;
        for (int w = 0; w < kGW; w++) {
            if (w < wave && c == cc)
                rank += wc[w][cc];
            t += wc[w][cc];
        }
        cnt[cc] = t;
    }
    return rank;
}

// Tile bytes: header, code records (8 * b each), one scale|position word per cell.
__device__ __forceinline__ uint32_t tile_bytes(const uint32_t cnt[4])
{
    const uint32_t codes = 8u * cnt[0] + 16u * cnt[1] + 32u * cnt[2] + 64u * cnt[3];
    const uint32_t cells = cnt[0] + cnt[1] + cnt[2] + cnt[3];
    return (kGHdr + codes + 4u * cells + 15u) & ~15u;
}

// One workgroup per tile: its size, into the offset table (16-byte units) or
// into the sizing statistics.
__global__ __launch_bounds__(kGT) void k_gsize(GPrep a)
{
    __shared__ uint32_t wc[kGW][4];
    const int kci = blockIdx.x, nbi = blockIdx.y;
    const Cell e = tile_cell(a, nbi, kci, threadIdx.x);
    uint32_t cnt[4];
    width_counts(e.c, wc, cnt);
    if (threadIdx.x == 0) {
        const uint32_t bytes = tile_bytes(cnt);
        if (a.table) {
            a.table[(uint64_t)nbi * a.kc + kci] = bytes / 16u;
        } else {
            atomicMax(a.stats, bytes);
            atomicAdd(reinterpret_cast<unsigned long long *>(a.stats + 2), (unsigned long long)(bytes / 16u));
        }
    }
}

// Exclusive scan of the tile sizes into offsets (16-byte units from the plan
// start; the tiles start at `base`), entry nt = the end of the last tile.
// If the tiles end past `cap` (16-byte units; a blob other than the one the
// plan was sized for), VBQ_STATUS_PLAN goes to *status and every entry is set
// to `base`, so nothing reads or writes past the buffer.  One workgroup of
// 1024 threads.
__global__ __launch_bounds__(1024) void k_gscan(uint32_t *table, uint32_t nt, uint32_t base, uint32_t cap,
                                                uint32_t *status)
{
    __shared__ uint32_t ws[16];
    __shared__ uint32_t carry;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    if (tid == 0)
        carry = base;
    __syncthreads();
    for (uint32_t i0 = 0; i0 < nt; i0 += 1024) {
        const uint32_t i = i0 + tid;
        const uint32_t v = i < nt ? table[i] : 0u;
        uint32_t inc = v;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d);
            if (lane >= d)
                inc += o;
        }
        if (lane == 63)
            ws[wave] = inc;
        __syncthreads();
        uint32_t before = carry;
        for (int w = 0; w < wave; w++)
            before += ws[w];
        if (i < nt)
            table[i] = before + inc - v;
        __syncthreads();
        if (tid == 1023)
            carry = before + inc;
        __syncthreads();
    }
    if (carry <= cap) {
        if (tid == 0)
            table[nt] = carry;
        return;
    }
    if (tid == 0 && status)
        atomicOr(status, VBQ_STATUS_PLAN);
    for (uint32_t i = tid; i <= nt; i += 1024)
        table[i] = base;
}

// One workgroup per tile: header, code records bucketed by width (8, 4, 2, 1;
// inside a bucket by column, then row), scale|position words in the same order.
__global__ __launch_bounds__(kGT) void k_gfill(GPrep a)
{
    __shared__ uint32_t wc[kGW][4];
    const int kci = blockIdx.x, nbi = blockIdx.y, u = threadIdx.x;
    const Cell e = tile_cell(a, nbi, kci, u);
    uint32_t cnt[4];
    const uint32_t rank = width_counts(e.c, wc, cnt);
    // a tile larger than the plan's largest, or a plan whose tiles did not fit
    // (the scan pointed them all at the first): write nothing (uniform)
    if (tile_bytes(cnt) > a.max_tile || (a.status && (*a.status & VBQ_STATUS_PLAN))) {
        if (u == 0 && a.status)
            atomicOr(a.status, VBQ_STATUS_PLAN);
        return;
    }
    uint8_t *t = a.buf + 16ull * a.table[(uint64_t)nbi * a.kc + kci];
    // buckets in the order 8, 4, 2, 1 bits
    uint32_t code_off[4], slot0[4];
    code_off[3] = kGHdr;
    slot0[3] = 0;
    code_off[2] = code_off[3] + 64u * cnt[3];
    slot0[2] = cnt[3];
    code_off[1] = code_off[2] + 32u * cnt[2];
    slot0[1] = slot0[2] + cnt[2];
    code_off[0] = code_off[1] + 16u * cnt[1];
    slot0[0] = slot0[1] + cnt[1];
    const uint32_t se_off = code_off[0] + 8u * cnt[0];
    if (e.c >= 0) {
        const uint32_t *row_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off);
        const uint32_t *slice_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off);
        const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
        const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.blob + a.off_scales);
        const uint64_t rs = (uint64_t)e.n * a.nS + (e.g >> 5);
        const WidthMasks wm = width_masks(wmap[2 * rs], wmap[2 * rs + 1], min(32, a.G - 32 * (e.g >> 5)));
        const uint64_t src =
            a.off_codes + (uint64_t)kRowPad * row_off[e.n] + slice_off[rs] + group_offset_in_slice(wm, e.c, e.g & 31);
        const U2 *s8 = reinterpret_cast<const U2 *>(a.blob + src);
        U2 *d8 = reinterpret_cast<U2 *>(t + code_off[e.c] + rank * (8u << e.c));
        for (int i = 0; i < (1 << e.c); i++)
            d8[i] = s8[i];
        const uint32_t sbits = scales[(uint64_t)e.n * a.G + e.g];
        reinterpret_cast<uint32_t *>(t + se_off)[slot0[e.c] + rank] = sbits | (uint32_t)u << 16;
    }
    if (u == 0) {
        const uint32_t bytes = tile_bytes(cnt);
        uint32_t *h = reinterpret_cast<uint32_t *>(t);
        h[0] = cnt[3] | cnt[2] << 16; // groups of width 8, 4
        h[1] = cnt[1] | cnt[0] << 16; // groups of width 2, 1
        h[2] = bytes;
        h[3] = se_off;
    }
}

// ---------------------------------------------------------------------------
// The GEMM kernel.

struct GArgs {
    const uint8_t *buf;  // GEMM plan
    const uint16_t *xp;  // [32 MT * token blocks][K] fp16, k-slot order (k_xpair)
    void *y;             // [M][ldy]
    float *part;         // K-split partial tiles (S > 1)
    uint32_t *ctr;       // K-split tickets, one per (row block, token block)
    int M, N, G, K, ldy;
    int nb, kc, S;
    int F;               // 1 KiB DMA copies per wave per tile (ring slot = 4 F KiB)
    int yt;
};

// Dequantize one 64-weight group of width B (code words cw, fp16 scale bits
// sb) into 32 pair words, stored four at a time to dst[0..7] (so that few of
// them are live at once): word j = fp16(s * (q_j - c)) | fp16(s * (q_{j+32} - c)) << 16,
// c = (2^B - 1) / 2, each product rounded once to nearest even.
template <int B>
__device__ __forceinline__ uint32_t code_pair(const uint32_t (&cw)[2 * B], int j)
{
    // 0x6400 | q is the fp16 value 1024 + q, for both halves
    constexpr uint32_t mask = (1u << B) - 1u;
    const int d = j / (16 / B), i = j % (16 / B);
    if constexpr (B == 8)
        return __builtin_amdgcn_perm(0x64646464u, cw[d], i ? 0x04030401u : 0x04020400u);
    else
        return ((cw[d] >> (B * i)) & (mask * 0x10001u)) | 0x64006400u;
}

template <int B>
__device__ __forceinline__ void dequant_group(const uint32_t (&cw)[2 * B], uint32_t sb, uint4 *dst)
{
    const _Float16 s = __builtin_bit_cast(_Float16, (uint16_t)sb);
    if constexpr (B == 1) {
        // q - c = -1/2 or +1/2: the weight is +-fp16(s / 2); its sign is
        // flipped where the code bit is 0
        const _Float16 hs = s * (_Float16)0.5f;
        const uint32_t base = (uint32_t)__builtin_bit_cast(uint16_t, hs) * 0x10001u;
#pragma unroll
        for (int d = 0; d < 2; d++) {
            const uint32_t nw = ~cw[d];
#pragma unroll
            for (int c4 = 0; c4 < 4; c4++) {
                uint32_t o[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    o[u] = base ^ ((nw << (15 - (4 * c4 + u))) & 0x80008000u);
                dst[4 * d + c4] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    } else {
        // h = 1024 + q.  For a finite s, s * h - (1024 + c) * s is one fp32
        // fma whose terms and result are exact (at most 23 significant bits),
        // so the only rounding is the conversion of s * (q - c) to fp16.  An
        // infinite s takes the exact fp16 steps (h - 1024) - c, then the product.
        constexpr float c = 0.5f * (float)((1u << B) - 1u);
        const float sf = (float)s;
        if (__builtin_isfinite(sf)) {
            const float t = -(1024.0f + c) * sf;
#pragma unroll
            for (int c4 = 0; c4 < 8; c4++) {
                uint32_t o[4];
#pragma unroll
                for (int u = 0; u < 4; u++) {
                    const hf2 v = u2h(code_pair<B>(cw, 4 * c4 + u));
                    hf2 w;
                    w.x = (_Float16)__builtin_fmaf((float)v.x, sf, t);
                    w.y = (_Float16)__builtin_fmaf((float)v.y, sf, t);
                    o[u] = h2u(w);
                }
                dst[c4] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        } else {
            const _Float16 k0 = (_Float16)-1024.0f, k1 = (_Float16)-c;
            const hf2 o0 = {k0, k0}, o1 = {k1, k1}, s2 = {s, s};
#pragma unroll
            for (int c4 = 0; c4 < 8; c4++) {
                uint32_t o[4];
#pragma unroll
                for (int u = 0; u < 4; u++)
                    o[u] = h2u(((u2h(code_pair<B>(cw, 4 * c4 + u)) + o0) + o1) * s2);
                dst[c4] = make_uint4(o[0], o[1], o[2], o[3]);
            }
        }
    }
}

// Pass lp of the width-B bucket of a tile in LDS: lane l dequantizes slot
// 64 lp + l (if the bucket has it) into row r, group gl of the W chunk.
template <int B>
__device__ __forceinline__ void dequant_pass(const uint8_t *tile, int lp, uint32_t cnt, uint32_t code_off,
                                             uint32_t slot0, uint32_t se_off, uint32_t *wchunk)
{
    const uint32_t s = (uint32_t)lp * 64u + (threadIdx.x & 63);
    if (s >= cnt)
        return;
    uint32_t cw[2 * B];
    const uint8_t *src = tile + code_off + s * (8u * B);
    if constexpr (B == 1) {
        const uint2 v = *reinterpret_cast<const uint2 *>(src);
        cw[0] = v.x;
        cw[1] = v.y;
    } else {
#pragma unroll
        for (int i = 0; i < B / 2; i++) {
            const uint4 v = reinterpret_cast<const uint4 *>(src)[i];
            cw[4 * i] = v.x;
            cw[4 * i + 1] = v.y;
            cw[4 * i + 2] = v.z;
            cw[4 * i + 3] = v.w;
        }
    }
    const uint32_t se = reinterpret_cast<const uint32_t *>(tile + se_off)[slot0 + s];
    const uint32_t r = (se >> 16) & (kBN - 1), gl = (se >> 23) & 1u;
    dequant_group<B>(cw, se & 0xffffu, reinterpret_cast<uint4 *>(wchunk + r * (kLdw / 2) + gl * 32u));
}

// The width buckets of a tile in a ring slot, from its header: pass p of the
// tile (64 groups of one width; the 8-bit passes first, then 4, 2, 1) is
// dequantized by dequant_one.
struct TileHdr {
    uint32_t c8, c4, c2, c1, se_off, o4, o2, o1;
    int b4, b2, b1, np; // first pass of the 4-, 2- and 1-bit buckets, pass count
};

__device__ __forceinline__ TileHdr tile_hdr(const uint8_t *tile)
{
    const uint4 h = *reinterpret_cast<const uint4 *>(tile);
    TileHdr t;
    t.c8 = h.x & 0xffffu;
    t.c4 = h.x >> 16;
    t.c2 = h.y & 0xffffu;
    t.c1 = h.y >> 16;
    t.se_off = h.w;
    t.o4 = kGHdr + 64u * t.c8;
    t.o2 = t.o4 + 32u * t.c4;
    t.o1 = t.o2 + 16u * t.c2;
    t.b4 = (int)((t.c8 + 63) >> 6);
    t.b2 = t.b4 + (int)((t.c4 + 63) >> 6);
    t.b1 = t.b2 + (int)((t.c2 + 63) >> 6);
    t.np = t.b1 + (int)((t.c1 + 63) >> 6);
    return t;
}

__device__ __forceinline__ void dequant_one(const uint8_t *tile, const TileHdr &t, int p, uint32_t *wchunk)
{
    if (p < t.b4)
        dequant_pass<8>(tile, p, t.c8, kGHdr, 0u, t.se_off, wchunk);
    else if (p < t.b2)
        dequant_pass<4>(tile, p - t.b4, t.c4, t.o4, t.c8, t.se_off, wchunk);
    else if (p < t.b1)
        dequant_pass<2>(tile, p - t.b2, t.c2, t.o2, t.c8 + t.c4, t.se_off, wchunk);
    else
        dequant_pass<1>(tile, p - t.b1, t.c1, t.o1, t.c8 + t.c4 + t.c2, t.se_off, wchunk);
}

// Every group of the tile in ring slot `tile` into the W chunk `wchunk`
// (wavefront w of the GEMM workgroup takes passes w, w + 8, ...).
__device__ __forceinline__ void dequant_tile(const uint8_t *tile, uint32_t *wchunk)
{
    const TileHdr t = tile_hdr(tile);
    for (int p = threadIdx.x >> 6; p < t.np; p += kMW)
        dequant_one(tile, t, p, wchunk);
}

// X in k-slot order: xp[m][64 g + 2 j + h] = x[m][64 g + j + 32 h] (j < 32),
// rows m < M only.  One thread per (row, group, 8 pairs); the first nctr
// threads also clear the K-split tickets of the GEMM launch that follows.
__global__ __launch_bounds__(256) void k_xpair(const uint16_t *__restrict__ x, int ldx, int M, int G,
                                               uint16_t *__restrict__ xp, int K, uint32_t *ctr, uint32_t nctr)
{
    const uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < nctr)
        ctr[i] = 0u;
    if (i >= (uint64_t)M * G * 4)
        return;
    const int o = (int)(i & 3), g = (int)((i >> 2) % (uint64_t)G), m = (int)(i / (4ull * G));
    const uint16_t *p = x + (uint64_t)m * ldx + 64 * g + 8 * o;
    const uint4 lo = *reinterpret_cast<const uint4 *>(p), hi = *reinterpret_cast<const uint4 *>(p + 32);
    const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w}, h[4] = {hi.x, hi.y, hi.z, hi.w};
    uint32_t w[8];
#pragma unroll
    for (int q = 0; q < 4; q++) {
        w[2 * q] = __builtin_amdgcn_perm(h[q], l[q], 0x05040100u);     // x_{2q} | x_{2q+32} << 16
        w[2 * q + 1] = __builtin_amdgcn_perm(h[q], l[q], 0x07060302u); // x_{2q+1} | x_{2q+33} << 16
    }
    uint4 *d = reinterpret_cast<uint4 *>(xp + (uint64_t)m * K + 64 * g + 16 * o);
    d[0] = make_uint4(w[0], w[1], w[2], w[3]);
    d[1] = make_uint4(w[4], w[5], w[6], w[7]);
}

// LDS-DMA of chunk c of the pair-ordered X rows m0 .. m0 + 32 MT - 1 into an X
// chunk (rows of kLdw halves, the last 8 not written): 1 KiB copies, copy i by
// wave i % 4; lanes beyond the chunk are masked.  Every wave issues exactly
// (9 MT + 3) / 4 copies (a copy past the last repeats an earlier one).
template <int MT>
__device__ __forceinline__ void dma_x(const uint16_t *xp, int K, int m0, int c, uint32_t dst)
{
    constexpr uint32_t bytes = 32u * MT * kLdw * 2u, nblk = (bytes + 1023u) / 1024u;
    constexpr int per = (int)((nblk + kGW - 1) / kGW);
    const int wave = threadIdx.x >> 6;
#pragma unroll
    for (int f = 0; f < per; f++) {
        uint32_t bi = (uint32_t)(f * kGW + wave);
        bi = bi < nblk ? bi : bi - nblk;
        const uint32_t o = bi * 1024u + (threadIdx.x & 63) * 16u;
        const uint32_t row = o / (kLdw * 2u), c16 = (o % (kLdw * 2u)) / 16u;
        const uint16_t *src = c16 < 16u ? xp + (uint64_t)(m0 + row) * K + 128u * c + 8u * c16 : xp;
        if (o < bytes)
            dma16(src, dst + bi * 1024u);
    }
}

// F copies of 1 KiB per wave: the tile at `src` (and whatever follows it, up
// to 4 F KiB; the plan ends with that much padding) into ring slot `dst`.
__device__ __forceinline__ void dma_tile(const uint8_t *src, uint32_t dst, int F)
{
    const int wave = threadIdx.x >> 6;
    const uint32_t lane16 = (threadIdx.x & 63) * 16u;
    for (int f = 0; f < F; f++) {
        const uint32_t o = (uint32_t)(f * kGW + wave) * 1024u;
        dma16(src + o + lane16, dst + o);
    }
}

template <int MT>
__global__ __launch_bounds__(kMT) void k_gemm(GArgs a)
{
    constexpr int BM = 32 * MT;
    // Eight wavefronts, two per SIMD: wavefront w runs the MFMAs of rows
    // 32 (w % 4) .. + 31 for token tiles t0 .. t0 + TW - 1 (the first half of
    // the tiles for w < 4, the second half for w >= 4; with one tile, only
    // w < 4), and every wavefront takes its share of the dequantization passes.
    // The LDS-DMA copies (and their waits) stay with wavefronts 0..3.
    constexpr int TW = MT > 1 ? MT / 2 : 1;
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t *wbuf = reinterpret_cast<uint32_t *>(smem);                          // [2][kBN][kLdw / 2] words
    uint32_t *xbuf = reinterpret_cast<uint32_t *>(smem + 2 * kWBytes);            // [2][BM][kLdw / 2] words
    uint8_t *ring = smem + 2 * kWBytes + 2 * BM * kLdw * 2;
    const uint32_t slot_bytes = 4096u * (uint32_t)a.F;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int rsl = wave & 3;                    // row slice of this wavefront's MFMAs
    const int t0 = MT > 1 ? (wave >> 2) * TW : 0; // its first token tile
    const bool mf = MT > 1 || wave < 4;          // it runs MFMAs
    const bool dma = wave < kGW;                 // it issues the LDS-DMA copies
    const int nbi = blockIdx.x, mbi = blockIdx.y, z = blockIdx.z;
    const int m0 = mbi * BM;
    const int kbeg = (int)((int64_t)z * a.kc / a.S), kend = (int)((int64_t)(z + 1) * a.kc / a.S);
    const int nk = kend - kbeg;
    // tile offsets of this split, entry i in lane i % 64 of toff[i / 64]
    const uint32_t *table = reinterpret_cast<const uint32_t *>(a.buf) + (uint64_t)nbi * a.kc + kbeg;
    uint32_t toff[4];
#pragma unroll
    for (int j = 0; j < 4; j++)
        toff[j] = lane + 64 * j < nk ? table[lane + 64 * j] : 0u;
    auto tile_src = [&](int k) -> const uint8_t * {
        const uint32_t v = k < 64 ? toff[0] : k < 128 ? toff[1] : k < 192 ? toff[2] : toff[3];
        return a.buf + 16ull * (uint32_t)__builtin_amdgcn_readlane((int)v, k & 63);
    };
    auto group_count = [&](int k) { return min(kTG, a.G - kTG * (kbeg + k)); };
    const uint32_t ring0 = lds_addr(ring);

    const uint32_t xbuf0 = lds_addr(xbuf);
    constexpr uint32_t xchunk = BM * kLdw * 2; // bytes of one X chunk

    // ---- prologue: tiles 0..2 in flight with the activations of chunk 0
    if (dma) {
        dma_x<MT>(a.xp, a.K, m0, kbeg, xbuf0);
        for (int k = 0; k < kRing && k < nk; k++)
            dma_tile(tile_src(k), ring0 + (uint32_t)k * slot_bytes, a.F);
        wait_vm0();
    }
    __syncthreads();
    dequant_tile(ring, wbuf);
    __syncthreads();

    f32x16 acc[TW];
#pragma unroll
    for (int t = 0; t < TW; t++)
#pragma unroll
        for (int r = 0; r < 16; r++)
            acc[t][r] = 0.f;

    for (int k = 0; k < nk; k++) {
        const int cur = k & 1;
        const bool more = k + 1 < nk, fetch = k + kRing < nk;
        if (more && dma) // into the X chunk of chunk k - 1, consumed before the last barrier
            dma_x<MT>(a.xp, a.K, m0, kbeg + k + 1, xbuf0 + (uint32_t)(cur ^ 1) * xchunk);
        if (fetch && dma) // into the slot of tile k, dequantized before the last barrier
            dma_tile(tile_src(k + kRing), ring0 + (uint32_t)(k % kRing) * slot_bytes, a.F);
        // ---- MFMAs of chunk k, with this wavefront's dequantization passes of
        // tile k + 1 between every second step, so that the matrix cores work
        // through the issued MFMAs while the same wavefront runs the passes'
        // vector instructions (the passes write the other W buffer)
        {
            const _Float16 *wb = reinterpret_cast<const _Float16 *>(wbuf + cur * (kWBytes / 4)) +
                                 (32 * rsl + (lane & 31)) * kLdw + 8 * (lane >> 5);
            const _Float16 *xb = reinterpret_cast<const _Float16 *>(xbuf + cur * (BM * kLdw / 2)) +
                                 (32 * t0 + (lane & 31)) * kLdw + 8 * (lane >> 5);
            const int steps = mf ? 4 * group_count(k) : 0;
            const uint8_t *ntile = ring + (uint32_t)((k + 1) % kRing) * slot_bytes;
            uint32_t *nw = wbuf + (cur ^ 1) * (kWBytes / 4);
            TileHdr th{};
            if (more)
                th = tile_hdr(ntile);
            int p = more ? wave : th.np; // this wavefront's next pass of tile k + 1
#pragma unroll
            for (int s = 0; s < 4 * kTG; s++) {
                if (s < steps) {
                    const int ko = (s >> 2) * 64 + (s & 3) * 16;
                    const hf8 b = *reinterpret_cast<const hf8 *>(wb + ko);
#pragma unroll
                    for (int t = 0; t < TW; t++) {
                        const hf8 xa = *reinterpret_cast<const hf8 *>(xb + t * 32 * kLdw + ko);
                        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(xa, b, acc[t], 0, 0, 0);
                    }
                }
                if ((s & 1) && p < th.np) {
                    dequant_one(ntile, th, p, nw);
                    p += kMW;
                }
            }
            for (; p < th.np; p += kMW)
                dequant_one(ntile, th, p, nw);
        }
        if (more && dma) {
            // everything but this iteration's tile copies: the activations of
            // chunk k + 1 and the tile of chunk k + 2
            if (fetch)
                wait_vm(a.F);
            else
                wait_vm0();
        }
        __syncthreads();
    }

    // ---- outputs: lane l, register r of this wavefront's token tile t0 + t
    // holds token 32 (t0 + t) + 8 (r / 4) + 4 (l / 32) + r % 4 of the block and
    // row 32 (w % 4) + l % 32
    const int nl = 32 * rsl + (lane & 31), n = nbi * kBN + nl;
    if (a.S == 1) {
        if (!mf)
            return;
#pragma unroll
        for (int t = 0; t < TW; t++)
#pragma unroll
            for (int r = 0; r < 16; r++) {
                const int m = m0 + 32 * (t0 + t) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < a.M && n < a.N) {
                    const uint64_t o = (uint64_t)m * a.ldy + n;
                    if (a.yt == VBQ_F16)
                        reinterpret_cast<__half *>(a.y)[o] = __float2half_rn(acc[t][r]);
                    else
                        reinterpret_cast<float *>(a.y)[o] = acc[t][r];
                }
            }
        return;
    }
    // K-split: this split's tile of partial sums, then the last split to
    // arrive adds the S tiles in split order and writes the outputs
    const int mb = gridDim.y;
    float *mine = a.part + (((uint64_t)z * mb + mbi) * a.nb + nbi) * (uint64_t)(BM * kBN);
    if (mf) {
#pragma unroll
        for (int t = 0; t < TW; t++)
#pragma unroll
            for (int r = 0; r < 16; r++)
                mine[(32 * (t0 + t) + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3)) * kBN + nl] = acc[t][r];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    __syncthreads();
    uint32_t *flag = xbuf; // the X chunks are no longer read
    if (tid == 0) {
        const uint32_t ticket =
            __hip_atomic_fetch_add(a.ctr + (uint64_t)mbi * a.nb + nbi, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        flag[0] = ticket;
    }
    __syncthreads();
    if (flag[0] != (uint32_t)a.S - 1u)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const float *p0 = a.part + ((uint64_t)mbi * a.nb + nbi) * (uint64_t)(BM * kBN);
    const uint64_t zstride = (uint64_t)mb * a.nb * (uint64_t)(BM * kBN);
    for (int i = tid; i < BM * kBN; i += kMT) {
        const int mi = i / kBN, ni = i % kBN;
        const int m = m0 + mi, nn = nbi * kBN + ni;
        float v = p0[i];
        for (int zz = 1; zz < a.S; zz++)
            v += __builtin_nontemporal_load(p0 + zz * zstride + i);
        if (m < a.M && nn < a.N) {
            const uint64_t o = (uint64_t)m * a.ldy + nn;
            if (a.yt == VBQ_F16)
                reinterpret_cast<__half *>(a.y)[o] = __float2half_rn(v);
            else
                reinterpret_cast<float *>(a.y)[o] = v;
        }
    }
    if (tid == 0)
        __hip_atomic_store(a.ctr + (uint64_t)mbi * a.nb + nbi, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Host side.

uint32_t lds_need(int MT, int F)
{
    return 2u * kWBytes + 2u * (32u * (uint32_t)MT) * kLdw * 2u + (uint32_t)kRing * 4096u * (uint32_t)F;
}

int gemm_cus() { return current_device_cus(); }

vbq_status check_gemm_plan(const vbq_gemm_plan *P)
{
    if (!P || P->magic != VBQ_GEMM_PLAN_MAGIC)
        return VBQ_ERR_LAYOUT;
    if (P->N < 1 || P->G < 1 || P->K != 64 * P->G || P->K > kMaxK || P->nb != (P->N + kBN - 1) / kBN ||
        P->kc != (P->G + kTG - 1) / kTG || P->slot_bytes < 4096 || P->slot_bytes % 4096 ||
        P->slot_bytes > 5 * 4096 || P->max_tile < kGHdr || P->max_tile > P->slot_bytes ||
        P->table_bytes != align_up(4ull * ((uint64_t)P->nb * P->kc + 1), 256) ||
        P->total_bytes < P->table_bytes + (uint64_t)P->slot_bytes)
        return VBQ_ERR_LAYOUT;
    return VBQ_OK;
}

GPrep gprep(const vbq_layout *L, const void *blob, int kc)
{
    GPrep a{};
    a.blob = (const uint8_t *)blob;
    a.off_row_off = L->off_row_off;
    a.off_slice_off = L->off_slice_off;
    a.off_wmap = L->off_wmap;
    a.off_scales = L->off_scales;
    a.off_codes = L->off_codes;
    a.N = (int)L->N;
    a.G = (int)L->G;
    a.nS = (int)L->nS;
    a.kc = kc;
    return a;
}

// Launch shape of a call: token tile (MT), token blocks, K-splits.
struct GShape {
    int MT, mb, S;
    uint32_t lds;
};

GShape gemm_shape(const vbq_gemm_plan *P, int M)
{
    const int F = P->slot_bytes / 4096;
    GShape s{};
    s.MT = M > 64 ? 4 : M > 32 ? 2 : 1;
    while (s.MT > 1 && lds_need(s.MT, F) > kGLds)
        s.MT /= 2;
    s.lds = lds_need(s.MT, F);
    s.mb = (M + 32 * s.MT - 1) / (32 * s.MT);
    // enough workgroups to cover the compute units, each K-split keeping at
    // least 8 chunks
    s.S = 1;
    const int cus = gemm_cus();
    const int64_t blocks = (int64_t)P->nb * s.mb;
    while (blocks * s.S < cus && (s.S + 1) * 8 <= P->kc && s.S < 16)
        s.S++;
    return s;
}

// Workspace of a call: K-split tickets, X in k-slot order (the rows of every
// token block; 256 bytes of padding for the last chunk of an odd G, which is
// copied whole), K-split partial tiles.
struct GWs {
    uint64_t nctr, xp, part, total;
};

GWs ws_layout(const vbq_gemm_plan *P, const GShape &s)
{
    GWs w{};
    w.nctr = s.S > 1 ? (uint64_t)P->nb * s.mb : 0;
    w.xp = align_up(4 * w.nctr, 256);
    const uint64_t rows = (uint64_t)s.mb * 32 * s.MT;
    w.part = align_up(w.xp + rows * (uint64_t)P->K * 2 + 256, 256);
    w.total = w.part + (s.S > 1 ? 4ull * s.S * s.mb * (uint64_t)P->nb * (32 * s.MT) * kBN : 0);
    return w;
}

template <int MT>
vbq_status launch_gemm(const GArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    VBQ_TRY(dynamic_lds_once((const void *)k_gemm<MT>, kGLds));
    hipLaunchKernelGGL(k_gemm<MT>, grid, dim3(kMT), lds, stream, a);
    return launch_status();
}

} // namespace

extern "C" {

vbq_status vbq_gemm_plan_init(const vbq_layout *L, const void *blob, vbq_gemm_plan *P, void *ws, size_t ws_bytes,
                              hipStream_t stream)
{
    if (!blob || !P)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if (!ws || ws_bytes < 16)
        return VBQ_ERR_WORKSPACE;
    if ((uintptr_t)blob % 256 || (uintptr_t)ws % 8)
        return VBQ_ERR_ALIGN;
    if (L->K > (uint32_t)kMaxK)
        return VBQ_ERR_SHAPE;
    vbq_gemm_plan p{};
    p.magic = VBQ_GEMM_PLAN_MAGIC;
    p.N = (int)L->N;
    p.K = (int)L->K;
    p.G = (int)L->G;
    p.nb = (p.N + kBN - 1) / kBN;
    p.kc = (p.G + kTG - 1) / kTG;
    p.table_bytes = align_up(4ull * ((uint64_t)p.nb * p.kc + 1), 256);
    VBQ_TRY(zero_words(ws, 16, stream));
    GPrep a = gprep(L, blob, p.kc);
    a.stats = (uint32_t *)ws;
    hipLaunchKernelGGL(k_gsize, dim3(p.kc, p.nb), dim3(kGT), 0, stream, a);
    VBQ_TRY(launch_status());
    uint32_t h[4];
    VBQ_TRY(hip_status(hipMemcpyAsync(h, ws, 16, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipStreamSynchronize(stream)));
    const uint64_t units = (uint64_t)h[2] | (uint64_t)h[3] << 32;
    p.max_tile = (int)h[0];
    p.slot_bytes = (int)align_up(h[0], 4096);
    // the kernel copies whole 4 KiB steps of the ring slot: padding after
    // the last tile keeps those copies inside the plan
    p.total_bytes = p.table_bytes + 16ull * units + (uint64_t)p.slot_bytes;
    if (p.table_bytes / 16 + units > 0xffffffffull)
        return VBQ_ERR_SHAPE;
    *P = p;
    return check_gemm_plan(P);
}

vbq_status vbq_gemm_prepare(const vbq_gemm_plan *P, const vbq_layout *L, const void *blob, void *buf,
                            uint32_t *status_word, hipStream_t stream)
{
    if (!blob || !buf)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    VBQ_TRY(check_gemm_plan(P));
    if ((int)L->N != P->N || (int)L->K != P->K)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)blob % 256 || (uintptr_t)buf % 256 || (uintptr_t)status_word % 4)
        return VBQ_ERR_ALIGN;
    VBQ_TRY(zero_words(buf, P->total_bytes, stream));
    if (status_word)
        VBQ_TRY(zero_words(status_word, 4, stream));
    GPrep a = gprep(L, blob, P->kc);
    a.buf = (uint8_t *)buf;
    a.table = (uint32_t *)buf;
    a.status = status_word;
    a.max_tile = (uint32_t)P->max_tile;
    const uint32_t nt = (uint32_t)P->nb * (uint32_t)P->kc;
    hipLaunchKernelGGL(k_gsize, dim3(P->kc, P->nb), dim3(kGT), 0, stream, a);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_gscan, dim3(1), dim3(1024), 0, stream, a.table, nt, (uint32_t)(P->table_bytes / 16),
                       (uint32_t)((P->total_bytes - (uint64_t)P->slot_bytes) / 16), status_word);
    VBQ_TRY(launch_status());
    hipLaunchKernelGGL(k_gfill, dim3(P->kc, P->nb), dim3(kGT), 0, stream, a);
    return launch_status();
}

vbq_status vbq_gemm_workspace(const vbq_gemm_plan *P, int M, size_t *bytes)
{
    if (!bytes)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_gemm_plan(P));
    if (M < 1 || M > kMaxGemmM)
        return VBQ_ERR_BATCH;
    *bytes = (size_t)ws_layout(P, gemm_shape(P, M)).total;
    return VBQ_OK;
}

vbq_status vbq_gemm(const vbq_gemm_plan *P, const void *buf, int M, const uint16_t *x, int ldx, void *y, int ldy,
                    vbq_dtype yt, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!buf || !x || !y || !ws)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_gemm_plan(P));
    if (M < 1 || M > kMaxGemmM)
        return VBQ_ERR_BATCH;
    if (ldx < P->K || ldy < P->N)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)buf % 256 || (uintptr_t)x % 16 || ldx % 8 || (uintptr_t)y % (yt == VBQ_F32 ? 4 : 2) ||
        (uintptr_t)ws % 256)
        return VBQ_ERR_ALIGN;
    const GShape s = gemm_shape(P, M);
    const GWs w = ws_layout(P, s);
    if (ws_bytes < w.total)
        return VBQ_ERR_WORKSPACE;
    uint8_t *wb = (uint8_t *)ws;
    GArgs a{};
    a.buf = (const uint8_t *)buf;
    a.xp = (const uint16_t *)(wb + w.xp);
    a.y = y;
    a.part = (float *)(wb + w.part);
    a.ctr = (uint32_t *)wb;
    a.M = M;
    a.N = P->N;
    a.G = P->G;
    a.K = P->K;
    a.ldy = ldy;
    a.nb = P->nb;
    a.kc = P->kc;
    a.S = s.S;
    a.F = P->slot_bytes / 4096;
    a.yt = (int)yt;
    const uint64_t items = std::max((uint64_t)M * P->G * 4, w.nctr);
    hipLaunchKernelGGL(k_xpair, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, x, ldx, M, P->G,
                       (uint16_t *)(wb + w.xp), P->K, a.ctr, (uint32_t)w.nctr);
    VBQ_TRY(launch_status());
    const dim3 grid((unsigned)P->nb, (unsigned)s.mb, (unsigned)s.S);
    switch (s.MT) {
    case 4: return launch_gemm<4>(a, grid, s.lds, stream);
    case 2: return launch_gemm<2>(a, grid, s.lds, stream);
    default: return launch_gemm<1>(a, grid, s.lds, stream);
    }
}

} // extern "C"
