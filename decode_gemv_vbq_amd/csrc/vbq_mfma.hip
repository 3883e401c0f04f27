// Batched decode GEMV on the matrix cores: Y[M][N] = X[M][K] W^T for up to 32
// tokens (one or two tiles of 16), read straight from a VBQ1 blob.
//
// "Variable Bit-width Quantization" (mlsanity.com page, Abstract) gives every
// 64-weight group its own width in {1, 2, 4, 8} and decodes with fused
// dequantize-and-multiply kernels.  With a decode batch of several tokens, one
// group's product is a 64-deep contraction that every token shares, so here
// each packed code is unpacked once per call and the multiply-accumulate runs
// on v_mfma_f32_16x16x32_f16.  A wavefront owns 16 weight rows; for each group
// column its 64 lanes unpack the 16 rows' groups into the B operand (row
// n = lane % 16, quarter q = lane / 16 of the group's 32 code pairs), while the
// A operand holds 16 tokens' activations of that group.  Lane (q, n) then
// holds the outputs of row n for tokens 4q..4q+3 of the tile; a second tile of
// 16 tokens reuses the same unpacked B operand with its own A and accumulator.
//
// Exactness.  An unpacked half is 2^(10-pos) + code exactly (the code lifted
// into the mantissa of a power of two) and the MFMA accumulates in fp32.  The
// offsets 2^(10-pos) + (2^b - 1)/2 are taken out by starting the accumulator at
// -sum_k x_k (2^(10-pos_k) + (2^b - 1)/2), one constant per (token, group,
// width) that the matrix cores compute from the staged activations.  The fp32
// group sum is multiplied by the group's fp16 scale (exact in fp32) and added
// in group order, which keeps the error inside the GEMV contract of vbq.h.
//
// K order inside a group: k-slot pair j of quarter q holds columns 8q+j and
// 8q+j+32, the order in which a code word carries its two halves (half 0 in the
// low 16 bits, half 1 in the high 16 bits).  A and B use the same order, and
// the contraction does not depend on it.
//
// Workgroup: 4 wavefronts = 64 rows x a K range of whole 4-group chunks, at
// most 128 registers per lane so that four workgroups (three with two token
// tiles, for the LDS) share a compute unit
// (four wavefronts per SIMD hide each other's LDS, matrix-core and memory
// latencies).  Per chunk, in one of two LDS buffers: the 4 groups' activations
// as fp16 pairs (wavefront w stages group w) and their offset constants.  The
// byte offset, width and scale of a row's 4 groups are worked out by the lanes
// (q, n) for group q of row n and handed to every lane of row n with the
// gfx950 lane swaps (v_permlane32_swap, v_permlane16_swap), in registers.
// While chunk c is computed, chunk c+1 is staged and its code words are loaded
// into registers, and the inputs of chunk c+2 (activations, width planes,
// slice offset, scale) are loaded.
//
// K segments.  A matrix with too few row blocks to fill the device has its
// chunks cut into segments (from the shape and the device's compute units
// alone).  With a large enough workspace each segment is its own workgroup,
// which writes fp32 partial sums that a second kernel adds in segment order;
// without one, a workgroup runs all segments and adds their sums in the same
// order.  Either way the result is the same, bit for bit.
#include "vbq_common.h"
#include "vbq_host.h"
#include "vbq_unpack.h"

#include <algorithm>

using namespace vbq;

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerBlock = 16 * kWaves;
constexpr int kChunk = 4;              // groups per chunk: wavefront w stages group w, lane (q, n) plans group q
constexpr int kTok = 144;              // LDS bytes per token of a staged group (128 + 16 against bank conflicts)
constexpr int kXGroup = 16 * kTok;     // one staged group, one tile of 16 tokens
constexpr int kCGroup = 4 * 16 * 4;    // offset constants of one group and tile: [width code][token] fp32
constexpr int kBufs = 2;
constexpr int kTabBytes = 5 * 48;      // B operands of the offset constants: [width code, or 4 = zero][Bm0 Bm1 Bo]
constexpr int kMaxSplits = 16;
constexpr int kMaxTiles = 2;           // token tiles of 16 per call

// Per token-tile count T (a call of up to 16 T tokens): one LDS buffer holds
// the chunk's activations [group][tile][token] and offset constants
// [group][tile][width][token].  One tile leaves room for four workgroups per
// compute unit, two tiles for three.
template <int T>
struct Geo {
    static constexpr int kXBytes = kChunk * T * kXGroup;
    static constexpr int kCBytes = kChunk * T * kCGroup;
    static constexpr int kBufBytes = kXBytes + kCBytes;
    static constexpr int kLdsBytes = kBufs * kBufBytes + kTabBytes;
    static constexpr int kBlocksPerCu = T == 1 ? 4 : 3;
};
static_assert(Geo<kMaxTiles>::kLdsBytes * Geo<kMaxTiles>::kBlocksPerCu <= 160 * 1024, "LDS of the resident workgroups");
constexpr uint32_t kNone = 0xffffffffu; // a buffer offset past every buffer: the load returns 0 and reads nothing

typedef _Float16 hf8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

struct MArgs {
    const uint8_t *blob;
    uint32_t blob_bytes;
    uint32_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    int N, G, nS, M;
    const uint16_t *x;
    uint32_t x_bytes;
    int ldx;
    void *y;
    int ldy, yt;
    float *part; // [splits][M][N] fp32 partial sums when splits > 1
    int splits, chunks_per_split;
    int seg;     // chunks per K segment (its sum is added to the total on its own)
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *p, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void *)p, 0, (int)bytes, 0x00020000);
}

// Mantissa position of k-slot pair j (0..7 of a quarter) for width code c.
__host__ __device__ constexpr int mpos(int c, int j)
{
    return c == 0 ? j : c == 1 ? 2 * (j & 3) : c == 2 ? 4 * (j & 1) : 0;
}

// fp16 pair (both halves) of -2^(10-pos) and of -(2^b - 1)/2.
__device__ __forceinline__ uint32_t neg_magic_pair(int pos) { return magic_pair(pos) | 0x80008000u; }
__device__ __forceinline__ uint32_t neg_offset_pair(int c)
{
    const uint32_t h = c == 0 ? 0xb800u : c == 1 ? 0xbe00u : c == 2 ? 0xc780u : 0xd7f8u; // -0.5 -1.5 -7.5 -127.5
    return h | (h << 16);
}

__device__ __forceinline__ hf8 as_hf8(uint32_t a, uint32_t b, uint32_t c, uint32_t d)
{
    const u32x4 v = {a, b, c, d};
    return __builtin_bit_cast(hf8, v);
}

// v of the lanes with the same n in rows (q) 0..3 of the wavefront, in every
// lane: v_permlane32_swap pairs rows 0,1 with 2,3 and v_permlane16_swap rows
// 0 with 1 and 2 with 3 (lane layout checked on the device).
__device__ __forceinline__ void rows4(uint32_t v, uint32_t (&o)[4])
{
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);       // [v0 v1 v0 v1], [v2 v3 v2 v3]
    const auto lo = __builtin_amdgcn_permlane16_swap(p[0], p[0], false, false); // v0, v1 in every row
    const auto hi = __builtin_amdgcn_permlane16_swap(p[1], p[1], false, false); // v2, v3 in every row
    o[0] = lo[0];
    o[1] = lo[1];
    o[2] = hi[0];
    o[3] = hi[1];
}

__device__ __forceinline__ f32x4 mfma(hf8 a, hf8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// The 8 k-slot pairs of quarter q of a group of width code C from the words
// loaded at the quarter's byte offset (b = 1: the word holding pairs 16*(q/2)
// .. +15, of which this quarter takes the byte rot/8 of each half; b = 2: one
// word; b = 4: two; b = 8: four).  Pair j = 2^(10-pos) + code in each half,
// pos = mpos(C, j).
template <int C>
__device__ __forceinline__ void unpack_quarter(const u32x4 &w, uint32_t rot, uint32_t *h)
{
    if constexpr (C == 0) {
        const uint32_t v = __builtin_amdgcn_alignbit(w.x, w.x, rot);
#pragma unroll
        for (int j = 0; j < 8; j++)
            h[j] = and_or(v, 0x00010001u << j, magic_pair(j));
    } else if constexpr (C == 1) {
        const uint32_t v = w.x, v8 = w.x >> 8;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            h[j] = and_or(v, 0x00030003u << (2 * j), magic_pair(2 * j));
            h[4 + j] = and_or(v8, 0x00030003u << (2 * j), magic_pair(2 * j));
        }
    } else if constexpr (C == 2) {
#pragma unroll
        for (int d = 0; d < 2; d++) {
            const uint32_t u = d ? w.y : w.x, u8 = u >> 8;
            h[4 * d] = and_or(u, 0x000f000fu, magic_pair(0));
            h[4 * d + 1] = and_or(u, 0x00f000f0u, magic_pair(4));
            h[4 * d + 2] = and_or(u8, 0x000f000fu, magic_pair(0));
            h[4 * d + 3] = and_or(u8, 0x00f000f0u, magic_pair(4));
        }
    } else {
#pragma unroll
        for (int d = 0; d < 4; d++) {
            const uint32_t u = d == 0 ? w.x : d == 1 ? w.y : d == 2 ? w.z : w.w;
            h[2 * d] = __builtin_amdgcn_perm(0x64646464u, u, 0x04020400u);     // bytes 0, 2: 1024 + code
            h[2 * d + 1] = __builtin_amdgcn_perm(0x64646464u, u, 0x04030401u); // bytes 1, 3
        }
    }
}

// Per-chunk inputs a lane loads one chunk before they are staged.
template <int T>
struct ChunkIn {
    u32x4 xa[T], xb[T]; // activations: token n + 16 t, columns 64g+8q..+7 and 64g+32+8q..+7 of the staged group
    uint32_t p0, p1;    // width-code bit planes of this lane's row in the slice of its planned group
    uint32_t so;        // slice offset in the row record
    uint32_t sc;        // scale of the planned group (fp16 bits)
};

template <int T>
__global__ __launch_bounds__(kThreads, Geo<T>::kBlocksPerCu) void k_gemv_mfma(MArgs a)
{
    constexpr int kXBytes = Geo<T>::kXBytes, kCBytes = Geo<T>::kCBytes, kBufBytes = Geo<T>::kBufBytes;
    extern __shared__ __align__(16) uint8_t smem[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15, q = lane >> 4;
    const int row = blockIdx.x * kRowsPerBlock + wave * 16 + n;
    const bool live = row < a.N;
    const int nch = (a.G + kChunk - 1) / kChunk;
    const int c0 = blockIdx.y * a.chunks_per_split;
    const int c1 = min(nch, c0 + a.chunks_per_split);
    const __amdgpu_buffer_rsrc_t rb = rsrc(a.blob, a.blob_bytes);
    const __amdgpu_buffer_rsrc_t rx = rsrc(a.x, a.x_bytes);
    uint8_t *tab = smem + kBufs * kBufBytes;

    // table of the offset constants' B operands: entry c < 4 is column width
    // code c (k-slot pairs 0..3, 4..7, then the (2^b - 1)/2 part), entry 4 zero
    if (threadIdx.x < 60) {
        const int c = threadIdx.x / 12, k = threadIdx.x % 12, v = k & 3;
        const uint32_t val = c == 4 ? 0u : k < 4 ? neg_magic_pair(mpos(c, v)) : k < 8 ? neg_magic_pair(mpos(c, 4 + v))
                                                                                      : neg_offset_pair(c);
        reinterpret_cast<uint32_t *>(tab)[threadIdx.x] = val;
    }

    const uint32_t row_off = __builtin_amdgcn_raw_buffer_load_b32(rb, live ? a.off_row_off + 4u * row : kNone, 0, 0);
    const uint32_t row_base = a.off_codes + 128u * row_off;

    // inputs of chunk ch (offsets kNone past the K range: zeros, no reads)
    auto load_in = [&](int ch, ChunkIn<T> &in) {
        const bool on = ch < c1;
        const int g = ch * kChunk + wave;
#pragma unroll
        for (int t = 0; t < T; t++) {
            const int tok = n + 16 * t;
            const bool xon = on && g < a.G && tok < a.M;
            const uint32_t xo = 2u * ((uint32_t)tok * (uint32_t)a.ldx + 64u * (uint32_t)g + 8u * q);
            in.xa[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, xon ? xo : kNone, 0, 0);
            in.xb[t] = __builtin_amdgcn_raw_buffer_load_b128(rx, xon ? xo + 64u : kNone, 0, 0);
        }
        const int gi = ch * kChunk + q;
        const bool mon = on && live && gi < a.G;
        const uint32_t rs = (uint32_t)row * (uint32_t)a.nS + (uint32_t)(gi >> 5);
        const u32x2 wm = __builtin_amdgcn_raw_buffer_load_b64(rb, mon ? a.off_wmap + 8u * rs : kNone, 0, 0);
        in.p0 = wm.x;
        in.p1 = wm.y;
        in.so = __builtin_amdgcn_raw_buffer_load_b32(rb, mon ? a.off_slice_off + 4u * rs : kNone, 0, 0);
        in.sc = __builtin_amdgcn_raw_buffer_load_b16(
            rb, mon ? a.off_scales + 2u * ((uint32_t)row * (uint32_t)a.G + (uint32_t)gi) : kNone, 0, 0);
    };

    // stage chunk ch into buffer bi (activations, offset constants); offs and
    // ms: the code offset | width and the width | scale << 16 of groups 0..3
    // of this lane's row
    auto stage = [&](int ch, int bi, const ChunkIn<T> &in, uint32_t (&offs)[4], uint32_t (&ms)[4]) {
        uint8_t *buf = smem + bi * kBufBytes;
        const u32x4 *tb = reinterpret_cast<const u32x4 *>(tab + 48 * (n < 4 ? n : 4));
        const u32x4 bm0 = tb[0], bm1 = tb[1], bo = tb[2];
#pragma unroll
        for (int t = 0; t < T; t++) {
            uint32_t p[8];
#pragma unroll
            for (int j = 0; j < 8; j++) {
                const uint32_t lo = in.xa[t][j >> 1], hi = in.xb[t][j >> 1];
                p[j] = __builtin_amdgcn_perm(hi, lo, (j & 1) ? 0x07060302u : 0x05040100u);
            }
            u32x4 *xs = reinterpret_cast<u32x4 *>(buf + (wave * T + t) * kXGroup + n * kTok + 32 * q);
            xs[0] = u32x4{p[0], p[1], p[2], p[3]};
            xs[1] = u32x4{p[4], p[5], p[6], p[7]};
            const hf8 A0 = as_hf8(p[0], p[1], p[2], p[3]), A1 = as_hf8(p[4], p[5], p[6], p[7]);
            f32x4 d = {0.f, 0.f, 0.f, 0.f};
            d = mfma(A0, as_hf8(bm0.x, bm0.y, bm0.z, bm0.w), d);
            d = mfma(A1, as_hf8(bm1.x, bm1.y, bm1.z, bm1.w), d);
            d = mfma(A0, as_hf8(bo.x, bo.y, bo.z, bo.w), d);
            d = mfma(A1, as_hf8(bo.x, bo.y, bo.z, bo.w), d);
            if (n < 4)
                *reinterpret_cast<f32x4 *>(buf + kXBytes + (wave * T + t) * kCGroup + n * 64 + 16 * q) = d;
        }

        const int gi = ch * kChunk + q, sl = gi >> 5, i = gi & 31;
        const int ng = min(32, a.G - 32 * sl);
        const WidthMasks wm = width_masks(in.p0, in.p1, ng);
        const int c = (int)(((in.p0 >> i) & 1u) | (((in.p1 >> i) & 1u) << 1));
        uint32_t start = 0u;
#pragma unroll
        for (int cc = 0; cc < 3; cc++)
            if (cc < c)
                start += (uint32_t)__popc(wm.m[cc]) << (3 + cc);
        const uint32_t rank = (uint32_t)__popc(pick4(wm.m, c) & ((1u << i) - 1u));
        const uint32_t off = row_base + in.so + start + (rank << (3 + c));
        const bool ok = live && ch < c1 && gi < a.G;
        // entry 0 (no group: a row past N, a chunk past the range) reads the
        // blob's first 16 bytes, which the scale 0 or the skipped group discards
        rows4(ok ? off | (uint32_t)c : 0u, offs);
        rows4(ok ? (uint32_t)c | (in.sc << 16) : 0u, ms);
    };

    // code words of the staged chunk in buffer bi, this lane's quarter (byte
    // offset (2q << c) & ~3 in the group: quarter q of a 1-bit group is the
    // half-word 2q of its words)
    const uint32_t qq = 2u * (uint32_t)q;
    auto load_codes = [&](const uint32_t (&offs)[4], u32x4 *cw) {
#pragma unroll
        for (int gl = 0; gl < kChunk; gl++) {
            const uint32_t e = offs[gl];
            const uint32_t off = (e & ~3u) + ((qq << (e & 3u)) & ~3u);
            cw[gl] = __builtin_amdgcn_raw_buffer_load_b128(rb, off, 0, 0);
        }
    };

    f32x4 acc[T], total[T];
#pragma unroll
    for (int t = 0; t < T; t++)
        acc[t] = total[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint32_t rot = 8u * (uint32_t)(q & 1);

    auto compute = [&](int ch, int bi, const u32x4 *cw, const uint32_t (&ms)[4]) {
        const uint8_t *buf = smem + bi * kBufBytes;
#pragma unroll
        for (int gl = 0; gl < kChunk; gl++) {
            if (ch < c1 && ch * kChunk + gl < a.G) { // uniform
                const uint32_t e = ms[gl];
                const int c = (int)(e & 3u);
                // the tiles' activations and offset constants first, so that
                // their LDS latency overlaps the unpack
                u32x4 x0[T], x1[T];
                f32x4 cinit[T];
#pragma unroll
                for (int t = 0; t < T; t++) {
                    const u32x4 *xs =
                        reinterpret_cast<const u32x4 *>(buf + (gl * T + t) * kXGroup + n * kTok + 32 * q);
                    x0[t] = xs[0];
                    x1[t] = xs[1];
                    cinit[t] =
                        *reinterpret_cast<const f32x4 *>(buf + kXBytes + (gl * T + t) * kCGroup + c * 64 + 16 * q);
                }
                uint32_t h[8];
                switch (c) {
                case 0: unpack_quarter<0>(cw[gl], rot, h); break;
                case 1: unpack_quarter<1>(cw[gl], rot, h); break;
                case 2: unpack_quarter<2>(cw[gl], rot, h); break;
                default: unpack_quarter<3>(cw[gl], rot, h); break;
                }
                const float s = (float)__builtin_bit_cast(_Float16, (uint16_t)(e >> 16));
                const hf8 B0 = as_hf8(h[0], h[1], h[2], h[3]), B1 = as_hf8(h[4], h[5], h[6], h[7]);
#pragma unroll
                for (int t = 0; t < T; t++) {
                    f32x4 d = mfma(as_hf8(x0[t].x, x0[t].y, x0[t].z, x0[t].w), B0, cinit[t]);
                    d = mfma(as_hf8(x1[t].x, x1[t].y, x1[t].z, x1[t].w), B1, d);
#pragma unroll
                    for (int r = 0; r < 4; r++)
                        acc[t][r] = __builtin_fmaf(s, d[r], acc[t][r]);
                }
            }
        }
        if (ch < c1 && (ch + 1 - c0) % a.seg == 0) { // end of a K segment (uniform)
#pragma unroll
            for (int t = 0; t < T; t++)
#pragma unroll
                for (int r = 0; r < 4; r++) {
                    total[t][r] += acc[t][r];
                    acc[t][r] = 0.f;
                }
        }
    };

    // ---- prologue: chunk c0 staged (buffer 0); its codes and the inputs of
    // chunk c0 + 1 in flight.  Then per step for chunk ch (buffer and register
    // set ch % 2): stage chunk ch+1, issue its codes and the inputs of ch+2,
    // compute chunk ch.  The loads are issued whether or not their chunk exists
    // (past the range they read nothing or a few bytes of the blob), so the
    // waits stay exact counts.
    ChunkIn<T> in;
    u32x4 cw0[kChunk], cw1[kChunk];
    uint32_t offs[4], ms0[4], ms1[4];
    load_in(c0, in);
    __syncthreads(); // the constant table
    stage(c0, 0, in, offs, ms0);
    load_codes(offs, cw0);
    load_in(c0 + 1, in);
    __syncthreads();
    for (int ch = c0; ch < c1; ch += 2) {
        stage(ch + 1, 1, in, offs, ms1);
        load_codes(offs, cw1);
        load_in(ch + 2, in);
        compute(ch, 0, cw0, ms0);
        __syncthreads();
        stage(ch + 2, 0, in, offs, ms0);
        load_codes(offs, cw0);
        load_in(ch + 3, in);
        compute(ch + 1, 1, cw1, ms1);
        __syncthreads();
    }

    if (!live)
        return;
#pragma unroll
    for (int tt = 0; tt < T; tt++)
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const int t = 16 * tt + 4 * q + r;
            if (t >= a.M)
                continue;
            const float v = total[tt][r] + acc[tt][r]; // acc is zero here unless the last segment is partial
            if (a.splits > 1) {
                a.part[((size_t)blockIdx.y * a.M + t) * a.N + row] = v;
            } else if (a.yt == VBQ_F32) {
                reinterpret_cast<float *>(a.y)[(size_t)t * a.ldy + row] = v;
            } else {
                reinterpret_cast<__half *>(a.y)[(size_t)t * a.ldy + row] = __float2half_rn(v);
            }
        }
}

// y[t][n] = 0 + part[0][t][n] + part[1][t][n] + ..., left to right: the
// order in which an unsplit workgroup adds its segment sums.
__global__ __launch_bounds__(256) void k_split_sum(const float *part, int splits, int M, int N, void *y, int ldy,
                                                   int yt)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i >= M * N)
        return;
    const int t = i / N, nn = i - t * N;
    float s = 0.f;
    for (int sp = 0; sp < splits; sp++)
        s += part[((size_t)sp * M + t) * N + nn];
    if (yt == VBQ_F32)
        reinterpret_cast<float *>(y)[(size_t)t * ldy + nn] = s;
    else
        reinterpret_cast<__half *>(y)[(size_t)t * ldy + nn] = __float2half_rn(s);
}

struct MfmaGeom {
    int blocks, splits, cps, seg;
    size_t ws; // workspace bytes the segments need as separate workgroups
};

// Row blocks x K segments: the segment count that minimizes (rounds of
// kBlocksPerCu workgroups per compute unit) x (chunks per segment + the
// start-up of a workgroup, about two chunks of latency), fewer segments on ties.
// The segments depend on the shape and the compute units only; they run as
// separate workgroups (splits) when ws_bytes holds their M*N fp32 partial sums
// each, else in one workgroup per row block.
int mfma_tiles(int M) { return M > 16 ? 2 : 1; }

MfmaGeom mfma_geom(const vbq_layout *L, int M, int cus, size_t ws_bytes)
{
    const int kBlocksPerCu = mfma_tiles(M) == 1 ? Geo<1>::kBlocksPerCu : Geo<2>::kBlocksPerCu;
    MfmaGeom g{};
    const int nch = ((int)L->G + kChunk - 1) / kChunk;
    g.blocks = ((int)L->N + kRowsPerBlock - 1) / kRowsPerBlock;
    int nseg = 1;
    g.seg = nch;
    constexpr int kStart = 2;
    const long slots = (long)cus * kBlocksPerCu;
    long best = (long)((g.blocks + slots - 1) / slots) * (nch + kStart);
    for (int s = 2; s <= std::min(kMaxSplits, nch); s++) {
        const int cps = (nch + s - 1) / s;
        if ((nch + cps - 1) / cps != s)
            continue; // s segments of cps chunks would leave one empty
        const long cost = (long)(((long)g.blocks * s + slots - 1) / slots) * (cps + kStart);
        if (cost < best) {
            best = cost;
            nseg = s;
            g.seg = cps;
        }
    }
    g.ws = nseg > 1 ? (size_t)nseg * M * L->N * 4 : 0;
    const bool split = nseg > 1 && ws_bytes >= g.ws;
    g.splits = split ? nseg : 1;
    g.cps = split ? g.seg : nch;
    return g;
}

} // namespace

namespace vbq {

bool mfma_applies(const vbq_layout *L, int M, const uint16_t *x, int ldx)
{
    return M >= 1 && M <= 16 * kMaxTiles && L->total_bytes < (1ull << 32) && (uintptr_t)x % 16 == 0 &&
           ldx % 8 == 0 && (uint64_t)(M - 1) * ldx * 2 + 2ull * L->K < (1ull << 32);
}

size_t mfma_workspace(const vbq_layout *L, int M)
{
    return mfma_geom(L, M, current_device_cus(), ~(size_t)0).ws;
}

vbq_status mfma_gemv(const GemvCall &g, void *ws, size_t ws_bytes)
{
    const vbq_layout *L = g.L;
    const MfmaGeom geo = mfma_geom(L, g.M, current_device_cus(), ws && (uintptr_t)ws % 4 == 0 ? ws_bytes : 0);
    MArgs a{};
    a.blob = (const uint8_t *)g.blob;
    a.blob_bytes = (uint32_t)L->total_bytes;
    a.off_row_off = (uint32_t)L->off_row_off;
    a.off_slice_off = (uint32_t)L->off_slice_off;
    a.off_wmap = (uint32_t)L->off_wmap;
    a.off_scales = (uint32_t)L->off_scales;
    a.off_codes = (uint32_t)L->off_codes;
    a.N = (int)L->N;
    a.G = (int)L->G;
    a.nS = (int)L->nS;
    a.M = g.M;
    a.x = g.x;
    a.x_bytes = (uint32_t)((uint64_t)(g.M - 1) * g.ldx * 2 + 2ull * L->K);
    a.ldx = g.ldx;
    a.y = g.y;
    a.ldy = g.ldy;
    a.yt = (int)g.yt;
    a.part = (float *)ws;
    a.splits = geo.splits;
    a.chunks_per_split = geo.cps;
    a.seg = geo.seg;
    if (mfma_tiles(g.M) == 1) {
        VBQ_TRY(dynamic_lds_once((const void *)k_gemv_mfma<1>, Geo<1>::kLdsBytes));
        hipLaunchKernelGGL(k_gemv_mfma<1>, dim3(geo.blocks, geo.splits), dim3(kThreads), Geo<1>::kLdsBytes, g.stream,
                           a);
    } else {
        VBQ_TRY(dynamic_lds_once((const void *)k_gemv_mfma<2>, Geo<2>::kLdsBytes));
        hipLaunchKernelGGL(k_gemv_mfma<2>, dim3(geo.blocks, geo.splits), dim3(kThreads), Geo<2>::kLdsBytes, g.stream,
                           a);
    }
    VBQ_TRY(launch_status());
    if (geo.splits > 1) {
        const int total = g.M * (int)L->N;
        hipLaunchKernelGGL(k_split_sum, dim3((total + 255) / 256), dim3(256), 0, g.stream, (const float *)ws,
                           geo.splits, g.M, (int)L->N, g.y, g.ldy, (int)g.yt);
        VBQ_TRY(launch_status());
    }
    return VBQ_OK;
}

} // namespace vbq
