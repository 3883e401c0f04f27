// Fused dequantize-and-multiply GEMV over the VBQ1 layout, M = 1..16 tokens.
//
// The decode path of "Variable Bit-width Quantization" (mlsanity.com page,
// Abstract): weights in contiguous 64-weight groups, each with its own width in
// {1,2,4,8}, read as packed codes and multiplied without ever materialising the
// dense matrix.  Decode is bound by memory bandwidth, so every byte of the
// packed stream is read exactly once, with wide loads, and the arithmetic is
// shaped to stay under that bound on CDNA4:
//
//  * A workgroup owns a tile of R rows x one K-slice of 32 groups (2048 K).
//    It stages the slice of x in LDS as fp16 pairs (x_p, x_{p+32}) per group,
//    XOR-swizzled by group so that lanes on different groups hit different
//    LDS bank groups.
//  * The R*32 groups of the tile are listed per width in LDS (a slot table
//    built from the width bit planes), so a wavefront always works on 64
//    groups of ONE width: no divergence between 1/2/4/8-bit paths.
//  * Lane = one group.  Each 32-bit code word is turned into fp16 pairs with a
//    single v_and_or_b32 (8-bit: v_perm_b32): the code field lands in the
//    mantissa of a power-of-two "magic" 2^(10-pos), so the half equals
//    2^(10-pos) + q exactly.  v_dot2_f32_f16 then multiplies two weights per
//    instruction with fp32 accumulation.  The magic offsets and the centre
//    (2^b-1)/2 are removed once per group through a per-(group, width)
//    constant computed from x during staging:
//        sum_j (q_j - c_b) x_j = acc - C_b,g,   C = sum_p magic_p (x_p + x_p+32) + c_b sum_j x_j
//    and the group's fp16 scale multiplies the difference.
//  * Per-group partials land in LDS and are summed per row in natural group
//    order (deterministic).  K > 2048 is split over slices; the last
//    workgroup of a row tile (atomic ticket) adds the slice partials in slice
//    order and writes y.  No MFMA: M <= 16 is not a dense contraction.
#include <stdio.h>

#include "vbq_common.h"
#include "vbq_host.h"

using namespace vbq;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxR = 32;
constexpr int kPsumStride = 33; // floats per psum row (pads away bank conflicts)

struct GemvArgs {
    const uint8_t *blob;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    int N, K, G, nS;
    int M;
    const uint16_t *x;
    int ldx;
    void *y;
    int ldy;
    int yt;
    float *partial;    // [nS][M][N] when nS > 1
    uint32_t *tickets; // [tiles] when nS > 1
    int R;             // rows per tile (<= 32)
};

// fp16 bits of 2^(10-pos), in both halves.
__host__ __device__ constexpr uint32_t magic_pair(int pos)
{
    return ((uint32_t)(25 - pos) << 10) | (((uint32_t)(25 - pos) << 10) << 16);
}

// Mantissa position used for pair i (inside its word) of a b-bit group, and
// the right shift applied to the word first.  Shared by the unpack and by the
// correction constants so the two can never disagree.
template <int B>
__host__ __device__ constexpr int pair_pos(int i)
{
    return B == 1 ? (i < 10 ? i : i - 10) : B == 2 ? (i <= 4 ? 2 * i : 2 * i - 10) : B == 4 ? (i <= 1 ? 4 * i : 4 * i - 8) : 0;
}
template <int B>
__host__ __device__ constexpr int pair_shift(int i)
{
    return B == 1 ? (i < 10 ? 0 : 10) : B == 2 ? (i <= 4 ? 0 : 10) : B == 4 ? (i <= 1 ? 0 : 8) : 0;
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// (w & mask) | magic in ONE v_and_or_b32.  Written out because gfx9 VOP3 has no
// literal operand and the compiler otherwise splits it into v_and + v_or with
// literals; here the mask sits in an SGPR and the magic in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic)
{
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
    return r;
}

// Turn the 2b code words of a b-bit group into 32 fp16 pairs (2^(10-pos)+q).
template <int B>
__device__ __forceinline__ void unpack_pairs(const uint32_t *w, uint32_t *h)
{
    if constexpr (B == 8) {
#pragma unroll
        for (int d = 0; d < 16; d++) {
            // bytes [b0, 0x64, b2, 0x64] and [b1, 0x64, b3, 0x64]: 1024 + q
            h[2 * d] = __builtin_amdgcn_perm(0x64646464u, w[d], 0x04020400u);
            h[2 * d + 1] = __builtin_amdgcn_perm(0x64646464u, w[d], 0x04030401u);
        }
    } else {
        constexpr int per = 16 / B;                // pairs per word
        constexpr uint32_t field = (1u << B) - 1u; // one code
#pragma unroll
        for (int d = 0; d < 2 * B; d++) {
#pragma unroll
            for (int i = 0; i < per; i++) {
                const int pos = pair_pos<B>(i);
                const int sh = pair_shift<B>(i);
                const uint32_t mask = (field | (field << 16)) << pos;
                h[d * per + i] = and_or(sh ? (w[d] >> sh) : w[d], mask, magic_pair(pos));
            }
        }
    }
}

template <int B>
__device__ __forceinline__ void load_codes(const uint8_t *__restrict__ p, uint32_t *w)
{
    if constexpr (B == 1) {
        U2 v = *reinterpret_cast<const U2 *>(p);
        w[0] = v.v[0];
        w[1] = v.v[1];
    } else {
#pragma unroll
        for (int k = 0; k < B / 2; k++) {
            U4 v = *reinterpret_cast<const U4 *>(p + 16 * k);
            w[4 * k + 0] = v.v[0];
            w[4 * k + 1] = v.v[1];
            w[4 * k + 2] = v.v[2];
            w[4 * k + 3] = v.v[3];
        }
    }
}

struct RowInfo {
    uint32_t p0, p1;   // width bit planes of this row-slice
    uint32_t base;     // row-slice record start, 8-byte units from the codes section
    uint16_t bb[4];    // bucket starts inside the slice record, 8-byte units
    uint16_t pre[4];   // slots of width c in earlier rows of the tile
};

// One pass: 64 slots of width B; lane = group.
template <int B, int MT>
__device__ __forceinline__ void run_pass(const GemvArgs &a, int slot, int nslots, const uint64_t *table,
                                         const uint32_t *xim, const float *corr, float *psum, int c,
                                         const uint8_t *codes)
{
    if (slot >= nslots)
        return;
    uint64_t e = table[slot];
    uint32_t lo = (uint32_t)e, hi = (uint32_t)(e >> 32);
    int g = (hi >> 16) & 0xff, r = hi >> 24;
    float s = __half2float(__ushort_as_half((unsigned short)(hi & 0xffffu)));
    uint32_t w[2 * B];
    load_codes<B>(codes + 8ull * lo, w);
    uint32_t h[32];
    unpack_pairs<B>(w, h);
    const int swz = g & 7;
#pragma unroll
    for (int m = 0; m < MT; m++) {
        if (m < a.M) {
            const uint32_t *xg = xim + (m * 32 + g) * 32;
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                U4 xv = *reinterpret_cast<const U4 *>(xg + ((k ^ swz) << 2));
                acc = dot2(h[4 * k + 0], xv.v[0], acc);
                acc = dot2(h[4 * k + 1], xv.v[1], acc);
                acc = dot2(h[4 * k + 2], xv.v[2], acc);
                acc = dot2(h[4 * k + 3], xv.v[3], acc);
            }
            float C = corr[(m * 4 + c) * 32 + g];
            psum[(m * kMaxR + r) * kPsumStride + g] = s * (acc - C);
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t *xim = reinterpret_cast<uint32_t *>(smem);                        // [MT][32][32] fp16 pairs
    float *corr = reinterpret_cast<float *>(xim + MT * 32 * 32);               // [MT][4][32]
    float *psum = corr + MT * 4 * 32;                                          // [MT][kMaxR][kPsumStride]
    uint64_t *table = reinterpret_cast<uint64_t *>(
        reinterpret_cast<uint8_t *>(psum) + ((MT * kMaxR * kPsumStride * 4 + 7) / 8) * 8); // [R*32]
    __shared__ RowInfo rows[kMaxR];
    __shared__ int s_total[4], s_tbase[5], s_pbase[5];
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int t = blockIdx.x, tile = blockIdx.y;
    const int R = a.R;
    const int n0 = tile * R;
    const int ng = min(32, a.G - 32 * t);
    const uint32_t *row_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off);
    const uint32_t *slice_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.blob + a.off_scales);
    const uint8_t *codes = a.blob + a.off_codes;

    // ---- phase 0a: per-row bucket counts and prefix sums (wave 0, lane = row)
    if (wave == 0) {
        int r = lane;
        int n = n0 + r;
        bool live = r < R && n < a.N;
        uint32_t p0 = 0, p1 = 0, base = 0;
        int cnt[4] = {0, 0, 0, 0};
        if (live) {
            uint64_t rs = (uint64_t)n * a.nS + t;
            p0 = wmap[2 * rs];
            p1 = wmap[2 * rs + 1];
            base = (uint32_t)((128ull * row_off[n] + slice_off[rs]) >> 3);
            WidthMasks m = width_masks(p0, p1, ng);
#pragma unroll
            for (int c = 0; c < 4; c++)
                cnt[c] = __popc(m.m[c]);
        }
        int incl[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            int v = cnt[c];
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                int u = __shfl_up(v, off, 64);
                if (lane >= off)
                    v += u;
            }
            incl[c] = v;
        }
        if (r < kMaxR) {
            RowInfo ri;
            ri.p0 = p0;
            ri.p1 = p1;
            ri.base = base;
            int bb = 0;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                ri.bb[c] = (uint16_t)bb;
                bb += cnt[c] << c;
                ri.pre[c] = (uint16_t)(incl[c] - cnt[c]);
            }
            rows[r] = ri;
        }
        if (lane == 63) {
            int tb = 0, pb = 0;
#pragma unroll
            for (int c = 0; c < 4; c++) {
                s_total[c] = incl[c];
                s_tbase[c] = tb;
                s_pbase[c] = pb;
                tb += incl[c];
                pb += (incl[c] + 63) / 64;
            }
            s_tbase[4] = tb;
            s_pbase[4] = pb;
        }
    }

    // ---- phase 0b: x slice -> LDS pairs (x_p, x_{p+32}), chunk k at k ^ (g & 7)
    for (int i = tid; i < a.M * ng * 32; i += kThreads) {
        int p = i & 31, g = (i >> 5) % ng, m = (i >> 5) / ng;
        const uint16_t *xs = a.x + (uint64_t)m * a.ldx + 64ull * (32 * t + g);
        uint32_t v = (uint32_t)xs[p] | ((uint32_t)xs[p + 32] << 16);
        xim[(m * 32 + g) * 32 + ((((p >> 2) ^ (g & 7)) << 2) | (p & 3))] = v;
    }
    __syncthreads();

    // ---- phase 0c: slot table (one entry per group of the tile)
    for (int i = tid; i < R * ng; i += kThreads) {
        int r = i / ng, gi = i % ng;
        int n = n0 + r;
        if (n >= a.N)
            continue;
        RowInfo ri = rows[r];
        WidthMasks m = width_masks(ri.p0, ri.p1, ng);
        int c = width_code(ri.p0, ri.p1, gi);
        int rank = __popc(pick4(m.m, c) & ((1u << gi) - 1u));
        uint32_t lo = ri.base + pick4(ri.bb, c) + ((uint32_t)rank << c);
        uint32_t sc = scales[(uint64_t)n * a.G + 32 * t + gi];
        uint32_t hi = sc | ((uint32_t)gi << 16) | ((uint32_t)r << 24);
        table[s_tbase[c] + pick4(ri.pre, c) + rank] = (uint64_t)lo | ((uint64_t)hi << 32);
    }

    // ---- phase 0d: correction constants C[m][c][g]
    for (int i = tid; i < a.M * ng * 4; i += kThreads) {
        int c = i & 3, g = (i >> 2) % ng, m = (i >> 2) / ng;
        const uint32_t *xg = xim + (m * 32 + g) * 32;
        float C = 0.f, X = 0.f;
#pragma unroll
        for (int p = 0; p < 32; p++) {
            uint32_t xv = xg[(((p >> 2) ^ (g & 7)) << 2) | (p & 3)];
            uint32_t mp;
            switch (c) {
            case 0: mp = magic_pair(pair_pos<1>(p & 15)); break;
            case 1: mp = magic_pair(pair_pos<2>(p & 7)); break;
            case 2: mp = magic_pair(pair_pos<4>(p & 3)); break;
            default: mp = 0x64006400u; break;
            }
            C = dot2(xv, mp, C);
            X = dot2(xv, 0x3c003c00u, X);
        }
        float cb = 0.5f * (float)((1 << (1 << c)) - 1);
        corr[(m * 4 + c) * 32 + g] = C + cb * X;
    }
    __syncthreads();

    // ---- phase 1: width-uniform passes, 64 groups each, spread over waves
    const int npass = s_pbase[4];
    for (int pi = wave; pi < npass; pi += kWaves) {
        int c = 0;
#pragma unroll
        for (int cc = 1; cc < 4; cc++)
            c += pi >= s_pbase[cc] ? 1 : 0;
        int slot = (pi - s_pbase[c]) * 64 + lane;
        const uint64_t *tb = table + s_tbase[c];
        switch (c) {
        case 0: run_pass<1, MT>(a, slot, s_total[0], tb, xim, corr, psum, 0, codes); break;
        case 1: run_pass<2, MT>(a, slot, s_total[1], tb, xim, corr, psum, 1, codes); break;
        case 2: run_pass<4, MT>(a, slot, s_total[2], tb, xim, corr, psum, 2, codes); break;
        default: run_pass<8, MT>(a, slot, s_total[3], tb, xim, corr, psum, 3, codes); break;
        }
    }
    __syncthreads();

    // ---- phase 2: per-row sums in natural group order
    const bool split = a.nS > 1;
    for (int i = tid; i < a.M * R; i += kThreads) {
        int m = i / R, r = i % R;
        int n = n0 + r;
        if (n >= a.N)
            continue;
        const float *ps = psum + (m * kMaxR + r) * kPsumStride;
        float v = 0.f;
        for (int g = 0; g < ng; g++)
            v += ps[g];
        if (split) {
            a.partial[((uint64_t)t * a.M + m) * a.N + n] = v;
        } else if (a.yt == VBQ_F16) {
            reinterpret_cast<__half *>(a.y)[(uint64_t)m * a.ldy + n] = __float2half_rn(v);
        } else {
            reinterpret_cast<float *>(a.y)[(uint64_t)m * a.ldy + n] = v;
        }
    }
    if (!split)
        return;

    // ---- phase 3: the last workgroup of this row tile adds the slices in order
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        uint32_t old = __hip_atomic_fetch_add(&a.tickets[tile], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        s_last = old == (uint32_t)(a.nS - 1);
    }
    __syncthreads();
    if (!s_last)
        return;
    __threadfence();
    for (int i = tid; i < a.M * R; i += kThreads) {
        int m = i / R, r = i % R;
        int n = n0 + r;
        if (n >= a.N)
            continue;
        float v = 0.f;
        for (int s = 0; s < a.nS; s++)
            v += a.partial[((uint64_t)s * a.M + m) * a.N + n];
        if (a.yt == VBQ_F16)
            reinterpret_cast<__half *>(a.y)[(uint64_t)m * a.ldy + n] = __float2half_rn(v);
        else
            reinterpret_cast<float *>(a.y)[(uint64_t)m * a.ldy + n] = v;
    }
    if (tid == 0)
        __hip_atomic_store(&a.tickets[tile], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

int tokens_template(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

size_t smem_bytes(int MT)
{
    size_t b = (size_t)MT * 32 * 32 * 4 + (size_t)MT * 4 * 32 * 4;
    b += (((size_t)MT * kMaxR * kPsumStride * 4 + 7) / 8) * 8;
    b += (size_t)kMaxR * 32 * 8;
    return b;
}

int rows_per_tile(const vbq_layout *L, int MT)
{
    // Enough workgroups to fill 256 CUs several times over, larger tiles when
    // the matrix allows (more groups per width bucket, fewer partial passes).
    uint64_t slices = L->nS;
    int R = 32;
    while (R > 8 && ((uint64_t)L->N + R - 1) / R * slices < 2048)
        R /= 2;
    (void)MT;
    return R;
}

template <int MT>
vbq_status launch(const GemvArgs &a, int tiles, hipStream_t stream)
{
    size_t sm = smem_bytes(MT);
    static bool configured = false;
    if (!configured) {
        VBQ_TRY(hip_status(hipFuncSetAttribute((const void *)k_gemv<MT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                               (int)sm)));
        configured = true;
    }
    hipLaunchKernelGGL(k_gemv<MT>, dim3(a.nS, tiles), dim3(kThreads), sm, stream, a);
    return launch_status();
}

uint64_t partial_bytes(const vbq_layout *L, int M) { return L->nS > 1 ? 4ull * L->nS * (uint64_t)M * L->N : 0; }

// One counter per row tile, sized for the smallest tile height (8 rows).
uint64_t ticket_bytes(const vbq_layout *L) { return align_up(4 * (((uint64_t)L->N + 7) / 8), 256); }

} // namespace

extern "C" {

vbq_status vbq_workspace_size(const vbq_layout *L, int M, size_t *bytes)
{
    if (!bytes)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    if (L->nS <= 1) {
        *bytes = 0;
        return VBQ_OK;
    }
    // [tickets | partials]: the tickets come first, at an offset that does not
    // depend on M, so one cleared workspace serves every M up to its size.
    *bytes = (size_t)(ticket_bytes(L) + align_up(partial_bytes(L, M), 256));
    return VBQ_OK;
}

vbq_status vbq_gemv_batched(const vbq_layout *L, const void *blob, int M, const uint16_t *x, int ldx, void *y, int ldy,
                            vbq_dtype yt, void *ws, size_t ws_bytes, hipStream_t stream)
{
    if (!blob || !x || !y)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    if (ldx < (int)L->K || ldy < (int)L->N)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)blob % 256 || (uintptr_t)x % 2 || (uintptr_t)y % (yt == VBQ_F32 ? 4 : 2))
        return VBQ_ERR_ALIGN;
    size_t need = 0;
    VBQ_TRY(vbq_workspace_size(L, M, &need));
    if (need && (!ws || ws_bytes < need))
        return VBQ_ERR_WORKSPACE;
    if (need && (uintptr_t)ws % 256)
        return VBQ_ERR_ALIGN;

    int MT = tokens_template(M);
    int R = rows_per_tile(L, MT);
    int tiles = (int)(((uint64_t)L->N + R - 1) / R);
    GemvArgs a;
    a.blob = (const uint8_t *)blob;
    a.off_row_off = L->off_row_off;
    a.off_slice_off = L->off_slice_off;
    a.off_wmap = L->off_wmap;
    a.off_scales = L->off_scales;
    a.off_codes = L->off_codes;
    a.N = (int)L->N;
    a.K = (int)L->K;
    a.G = (int)L->G;
    a.nS = (int)L->nS;
    a.M = M;
    a.x = x;
    a.ldx = ldx;
    a.y = y;
    a.ldy = ldy;
    a.yt = (int)yt;
    a.tickets = need ? (uint32_t *)ws : nullptr;
    a.partial = need ? (float *)((uint8_t *)ws + ticket_bytes(L)) : nullptr;
    a.R = R;
    switch (MT) {
    case 1: return launch<1>(a, tiles, stream);
    case 2: return launch<2>(a, tiles, stream);
    case 4: return launch<4>(a, tiles, stream);
    case 8: return launch<8>(a, tiles, stream);
    default: return launch<16>(a, tiles, stream);
    }
}

vbq_status vbq_gemv(const vbq_layout *L, const void *blob, const uint16_t *x, void *y, vbq_dtype yt, void *ws,
                    size_t ws_bytes, hipStream_t stream)
{
    if (!L)
        return VBQ_ERR_INVALID_ARG;
    return vbq_gemv_batched(L, blob, 1, x, (int)L->K, y, (int)L->N, yt, ws, ws_bytes, stream);
}

} // extern "C"
