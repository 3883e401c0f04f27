// Fused dequantize-and-multiply GEMV over the VBQ1 layout, M = 1..16 tokens.
//
// The decode path of "Variable Bit-width Quantization" (mlsanity.com page,
// Abstract): weights in contiguous 64-weight groups, each with its own width in
// {1,2,4,8}, read as packed codes and multiplied without ever materialising the
// dense matrix.  Decode is bound by memory bandwidth, so every packed byte is
// read exactly once and the arithmetic is shaped to stay under that bound:
//
//  * Persistent workgroups own whole rows (no split-K, hence no cross-workgroup
//    traffic or fences).  Each stages x once as fp16 pairs (x_p, x_{p+32}) per
//    group in LDS, XOR-swizzled by group so lanes on different groups hit
//    different LDS bank groups, then walks its row tiles.
//  * A unit = R rows x SG K-slices.  Its groups are listed per width in an LDS
//    slot table built from the width bit planes, so a wavefront always works on
//    64 groups of ONE width: no divergence between the 1/2/4/8-bit paths.
//  * Lane = one group.  Each 32-bit code word becomes fp16 pairs with a single
//    v_and_or_b32 (8-bit: v_perm_b32): the code field lands in the mantissa of
//    a power-of-two "magic" 2^(10-pos), so each half equals 2^(10-pos) + q
//    exactly, and v_dot2_f32_f16 multiplies two weights per instruction into
//    an fp32 accumulator.  The magic offsets and the centre (2^b-1)/2 are
//    removed once per group with a per-(group, width) constant of x:
//        sum_j (q_j - c_b) x_j = acc - C,  C = sum_p magic_p (x_p + x_{p+32}) + c_b sum_j x_j
//    and the group's fp16 scale multiplies the difference.
//  * Code loads of the next pass are issued before the current pass computes,
//    and the next unit's tables are fetched while this unit computes.
//  * Per-group partials are summed per row in natural group order, units in
//    K order: the result does not depend on the launch shape's timing.
//  * No MFMA: M <= 16 tokens is not a dense contraction.
#include <stdio.h>

#include <algorithm>

#include "vbq_common.h"
#include "vbq_host.h"
#include "vbq_unpack.h"

using namespace vbq;

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kMaxRS = 64;    // row-slices per unit (one wave lane each)
constexpr int kMaxRows = 32;  // rows per tile

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
    int R;        // rows per tile (<= 32)
    int SG;       // K-slices per unit (R * SG <= 64, R * SG * 32 <= slot capacity)
    int CHK;      // K-slices of x resident in LDS at a time
    int tiles;    // ceil(N / R)
    int slots;    // slot-table capacity
};

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

// One row-slice of the current unit, as seen by the slot-table build.
struct RowSlice {
    uint32_t p0, p1;  // width bit planes
    uint32_t base;    // record start of this row-slice, 8-byte units from the codes section
    uint16_t bb[4];   // bucket starts inside the row-slice record, 8-byte units
    uint16_t pre[4];  // slots of width c in earlier row-slices of the unit
};

// Work unit of a workgroup: rows [tile*R, tile*R + R) x slices [t0, t0 + ns).
struct Unit {
    int tile, t0, ns;
};

__device__ __forceinline__ bool unit_valid(const Unit &u, const GemvArgs &a) { return u.tile < a.tiles; }

__device__ __forceinline__ Unit first_unit(const GemvArgs &a)
{
    Unit u;
    u.tile = blockIdx.x;
    u.t0 = 0;
    u.ns = min(a.SG, min(a.CHK, a.nS));
    return u;
}

// Units run slice-group by slice-group inside an x chunk, chunks in order,
// then the next row tile of this workgroup.
__device__ __forceinline__ Unit next_unit(const Unit &u, const GemvArgs &a)
{
    Unit n = u;
    int t = u.t0 + u.ns;
    if (t >= a.nS) {
        n.tile = u.tile + gridDim.x;
        t = 0;
    }
    int chunk_end = min(a.nS, (t / a.CHK + 1) * a.CHK);
    n.t0 = t;
    n.ns = min(a.SG, chunk_end - t);
    return n;
}

// Metadata of one unit held in registers until the slot table is built.
struct UnitMeta {
    uint32_t p0, p1, row_off, slice_off; // lane-owned row-slice (wave 0)
    uint32_t scale[4];                   // up to 4 group items per thread
};

template <int MT>
__device__ __forceinline__ void fetch_meta(const Unit &u, const GemvArgs &a, UnitMeta &m)
{
    const int tid = threadIdx.x;
    m.p0 = m.p1 = m.row_off = m.slice_off = 0;
    if (!unit_valid(u, a))
        return;
    const uint32_t *row_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off);
    const uint32_t *slice_off = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.blob + a.off_scales);
    const int n0 = u.tile * a.R;
    if (tid < a.R * u.ns) {
        int r = tid / u.ns, s = tid % u.ns;
        int n = n0 + r;
        if (n < a.N) {
            uint64_t rs = (uint64_t)n * a.nS + u.t0 + s;
            m.p0 = wmap[2 * rs];
            m.p1 = wmap[2 * rs + 1];
            m.row_off = row_off[n];
            m.slice_off = slice_off[rs];
        }
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
        int i = tid + k * kThreads; // item = (row-slice, group in slice)
        int l = i >> 5, gi = i & 31;
        int r = l / u.ns, s = l % u.ns;
        int n = n0 + r;
        int g = 32 * (u.t0 + s) + gi;
        m.scale[k] = 0;
        if (l < a.R * u.ns && n < a.N && g < a.G)
            m.scale[k] = scales[(uint64_t)n * a.G + g];
    }
}

// Stage x for slices [t0, t0 + ns) of the chunk as swizzled pairs, then the
// per-(token, group, width) corrections.
template <int MT>
__device__ void stage_x(const GemvArgs &a, int t0, int ns, uint32_t *xim, float *corr)
{
    const int tid = threadIdx.x;
    const int CHG = a.CHK * 32;
    const int gch = min(ns * 32, a.G - 32 * t0);
    for (int i = tid; i < a.M * gch * 32; i += kThreads) {
        int p = i & 31, g = (i >> 5) % gch, m = (i >> 5) / gch;
        const uint16_t *xs = a.x + (uint64_t)m * a.ldx + 64ull * (32 * t0 + g);
        uint32_t v = (uint32_t)xs[p] | ((uint32_t)xs[p + 32] << 16);
        xim[(m * CHG + g) * 32 + ((((p >> 2) ^ (g & 7)) << 2) | (p & 3))] = v;
    }
    __syncthreads();
    // C_b = sum_p magic_b(p) (x_p + x_{p+32}) + c_b sum_j x_j, where magic_b(p)
    // depends on p only through p mod 16/8/4 for b = 1/2/4 (and is 1024 for b = 8).
    for (int i = tid; i < a.M * gch; i += kThreads) {
        int g = i % gch, m = i / gch;
        const uint32_t *xg = xim + (m * CHG + g) * 32;
        float X2[32];
#pragma unroll
        for (int p = 0; p < 32; p++)
            X2[p] = dot2(xg[(((p >> 2) ^ (g & 7)) << 2) | (p & 3)], 0x3c003c00u, 0.f);
        float S16[16], S8[8], S4[4];
#pragma unroll
        for (int j = 0; j < 16; j++)
            S16[j] = X2[j] + X2[j + 16];
#pragma unroll
        for (int j = 0; j < 8; j++)
            S8[j] = S16[j] + S16[j + 8];
#pragma unroll
        for (int j = 0; j < 4; j++)
            S4[j] = S8[j] + S8[j + 4];
        float C0 = 0.f, C1 = 0.f, C2 = 0.f;
#pragma unroll
        for (int j = 0; j < 16; j++)
            C0 = fmaf((float)(1 << (10 - pair_pos<1>(j))), S16[j], C0);
#pragma unroll
        for (int j = 0; j < 8; j++)
            C1 = fmaf((float)(1 << (10 - pair_pos<2>(j))), S8[j], C1);
#pragma unroll
        for (int j = 0; j < 4; j++)
            C2 = fmaf((float)(1 << (10 - pair_pos<4>(j))), S4[j], C2);
        float X = (S4[0] + S4[1]) + (S4[2] + S4[3]);
        float4 cv = make_float4(fmaf(0.5f, X, C0), fmaf(1.5f, X, C1), fmaf(7.5f, X, C2), fmaf(127.5f, X, 1024.f * X));
        *reinterpret_cast<float4 *>(corr + (m * CHG + g) * 4) = cv;
    }
    __syncthreads();
}

// Pending pass: the lane's table entry and its loaded code words.
struct Pending {
    int c;          // width code of the pass (wave-uniform), -1 when none
    bool live;      // lane has a slot
    uint32_t lo, hi;
    U4 w[4];
};

__device__ __forceinline__ int pass_width(int pi, const int *pbase)
{
    int c = 0;
#pragma unroll
    for (int cc = 1; cc < 4; cc++)
        c += pi >= pbase[cc] ? 1 : 0;
    return c;
}

__device__ __forceinline__ void issue_pass(Pending &p, int pi, int npass, const int *pbase, const int *tbase,
                                           const int *total, const uint64_t *table, const uint8_t *codes)
{
    const int lane = threadIdx.x & 63;
    p.c = -1;
    p.live = false;
    if (pi >= npass)
        return;
    int c = pass_width(pi, pbase);
    int slot = (pi - pbase[c]) * 64 + lane;
    p.c = c;
    p.live = slot < total[c];
    if (!p.live)
        return;
    uint64_t e = table[tbase[c] + slot];
    p.lo = (uint32_t)e;
    p.hi = (uint32_t)(e >> 32);
    const uint8_t *src = codes + 8ull * p.lo;
    switch (c) {
    case 0: {
        U2 v = *reinterpret_cast<const U2 *>(src);
        p.w[0].v[0] = v.v[0];
        p.w[0].v[1] = v.v[1];
        break;
    }
    case 1: p.w[0] = *reinterpret_cast<const U4 *>(src); break;
    case 2:
        p.w[0] = *reinterpret_cast<const U4 *>(src);
        p.w[1] = *reinterpret_cast<const U4 *>(src + 16);
        break;
    default:
#pragma unroll
        for (int k = 0; k < 4; k++)
            p.w[k] = *reinterpret_cast<const U4 *>(src + 16 * k);
        break;
    }
}

template <int B, int MT>
__device__ __forceinline__ void compute_slot(const Pending &p, const GemvArgs &a, const uint32_t *xim,
                                             const float *corr, float *psum, int gbase, int pstride, int prow)
{
    uint32_t w[2 * B];
#pragma unroll
    for (int d = 0; d < 2 * B; d++)
        w[d] = p.w[d / 4].v[d % 4];
    uint32_t h[32];
    unpack_pairs<B>(w, h);
    const int gl = (p.hi >> 16) & 0xff, r = p.hi >> 24;
    const int g = gbase + gl;
    const float s = __half2float(__ushort_as_half((unsigned short)(p.hi & 0xffffu)));
    const int CHG = a.CHK * 32;
    const int swz = g & 7;
#pragma unroll
    for (int m = 0; m < MT; m++) {
        if (m < a.M) {
            const uint32_t *xg = xim + (m * CHG + g) * 32;
            float acc = 0.f;
#pragma unroll
            for (int k = 0; k < 8; k++) {
                U4 xv = *reinterpret_cast<const U4 *>(xg + ((k ^ swz) << 2));
                acc = dot2(h[4 * k + 0], xv.v[0], acc);
                acc = dot2(h[4 * k + 1], xv.v[1], acc);
                acc = dot2(h[4 * k + 2], xv.v[2], acc);
                acc = dot2(h[4 * k + 3], xv.v[3], acc);
            }
            float C = corr[(m * CHG + g) * 4 + (B == 1 ? 0 : B == 2 ? 1 : B == 4 ? 2 : 3)];
            psum[m * pstride + r * prow + gl] = s * (acc - C);
        }
    }
}

template <int MT>
__global__ __launch_bounds__(kThreads) void k_gemv(GemvArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int CHG = a.CHK * 32;
    uint32_t *xim = reinterpret_cast<uint32_t *>(smem);             // [MT][CHG][32] fp16 pairs
    float *corr = reinterpret_cast<float *>(xim + MT * CHG * 32);   // [MT][CHG][4]
    uint64_t *table = reinterpret_cast<uint64_t *>(corr + MT * CHG * 4); // [slots]
    float *psum = reinterpret_cast<float *>(table + a.slots);      // [MT][R][SG*32 + 1]
    __shared__ RowSlice rsl[kMaxRS];
    __shared__ float acc_tile[MT][kMaxRows];
    __shared__ int s_total[4], s_tbase[4], s_pbase[5];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint8_t *codes = a.blob + a.off_codes;
    const int prow = a.SG * 32 + 1;
    const int pstride = a.R * prow;

    Unit u = first_unit(a);
    UnitMeta meta;
    fetch_meta<MT>(u, a, meta);
    int staged = -1;

    while (unit_valid(u, a)) {
        const Unit nu = next_unit(u, a);
        const int n0 = u.tile * a.R;
        const int chunk = u.t0 / a.CHK;
        if (chunk != staged) {
            __syncthreads(); // previous readers of xim/corr are done
            stage_x<MT>(a, chunk * a.CHK, min(a.CHK, a.nS - chunk * a.CHK), xim, corr);
            staged = chunk;
        }
        // acc_tile[m][r] belongs to thread 32*(m*R + r) (the row's reducing lane 0)
        if (u.t0 == 0) {
            for (int i = tid >> 5; i < a.M * a.R; i += kThreads / 32)
                if ((tid & 31) == 0)
                    acc_tile[i / a.R][i % a.R] = 0.f;
        }

        // ---- slot table, part 1: per row-slice counts and prefix sums (wave 0)
        if (wave == 0) {
            const int nrs = a.R * u.ns;
            bool live = lane < nrs && n0 + lane / u.ns < a.N;
            int s = lane % u.ns;
            int ng = max(0, min(32, a.G - 32 * (u.t0 + s)));
            int cnt[4] = {0, 0, 0, 0};
            WidthMasks wm = width_masks(meta.p0, meta.p1, ng);
            if (live) {
#pragma unroll
                for (int c = 0; c < 4; c++)
                    cnt[c] = __popc(wm.m[c]);
            }
            int incl[4];
#pragma unroll
            for (int c = 0; c < 4; c++) {
                int v = cnt[c];
#pragma unroll
                for (int off = 1; off < 64; off <<= 1) {
                    int t = __shfl_up(v, off, 64);
                    if (lane >= off)
                        v += t;
                }
                incl[c] = v;
            }
            if (lane < nrs) {
                RowSlice rs;
                rs.p0 = live ? meta.p0 : 0u;
                rs.p1 = live ? meta.p1 : 0u;
                rs.base = (uint32_t)((128ull * meta.row_off + meta.slice_off) >> 3);
                int bb = 0;
#pragma unroll
                for (int c = 0; c < 4; c++) {
                    rs.bb[c] = (uint16_t)bb;
                    bb += cnt[c] << c;
                    rs.pre[c] = (uint16_t)(incl[c] - cnt[c]);
                }
                rsl[lane] = rs;
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
                s_pbase[4] = pb;
            }
        }
        __syncthreads();

        // ---- slot table, part 2: one entry per group (width-major, then row-slice, then g)
#pragma unroll
        for (int k = 0; k < 4; k++) {
            int i = tid + k * kThreads;
            int l = i >> 5, gi = i & 31;
            if (l >= a.R * u.ns)
                continue;
            int r = l / u.ns, s = l % u.ns;
            if (n0 + r >= a.N || 32 * (u.t0 + s) + gi >= a.G)
                continue;
            RowSlice rs = rsl[l];
            int ng = min(32, a.G - 32 * (u.t0 + s));
            WidthMasks wm = width_masks(rs.p0, rs.p1, ng);
            int c = width_code(rs.p0, rs.p1, gi);
            int rank = __popc(pick4(wm.m, c) & ((1u << gi) - 1u));
            uint32_t lo = rs.base + pick4(rs.bb, c) + ((uint32_t)rank << c);
            uint32_t gl = (uint32_t)(32 * s + gi);
            uint32_t hi = (meta.scale[k] & 0xffffu) | (gl << 16) | ((uint32_t)r << 24);
            table[s_tbase[c] + pick4(rs.pre, c) + rank] = (uint64_t)lo | ((uint64_t)hi << 32);
        }
        __syncthreads();

        // ---- next unit's metadata in flight while this unit computes
        fetch_meta<MT>(nu, a, meta);

        // ---- passes: 64 groups of one width each; loads one pass ahead
        const int npass = s_pbase[4];
        const int gbase = (u.t0 - chunk * a.CHK) * 32;
        int pb[5], tb[4], tot[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            pb[c] = s_pbase[c];
            tb[c] = s_tbase[c];
            tot[c] = s_total[c];
        }
        pb[4] = npass;
        Pending cur, nxt;
        int pi = wave;
        issue_pass(cur, pi, npass, pb, tb, tot, table, codes);
        while (pi < npass) {
            issue_pass(nxt, pi + kWaves, npass, pb, tb, tot, table, codes);
            if (cur.live) {
                switch (cur.c) {
                case 0: compute_slot<1, MT>(cur, a, xim, corr, psum, gbase, pstride, prow); break;
                case 1: compute_slot<2, MT>(cur, a, xim, corr, psum, gbase, pstride, prow); break;
                case 2: compute_slot<4, MT>(cur, a, xim, corr, psum, gbase, pstride, prow); break;
                default: compute_slot<8, MT>(cur, a, xim, corr, psum, gbase, pstride, prow); break;
                }
            }
            cur = nxt;
            pi += kWaves;
        }
        __syncthreads();

        // ---- row sums of this unit: 32 lanes per row, fixed order (lane j adds
        // groups j, j+32, ...; then a fixed butterfly), units added in K order
        const int gcount = min(u.ns * 32, a.G - 32 * u.t0);
        const bool last = u.t0 + u.ns >= a.nS;
        for (int i = tid >> 5; i < ((a.M * a.R + 7) & ~7); i += kThreads / 32) {
            const int j = tid & 31;
            const int m = i / a.R, r = i % a.R;
            const bool row_live = i < a.M * a.R && n0 + r < a.N;
            float v = 0.f;
            if (row_live) {
                const float *ps = psum + m * pstride + r * prow;
                for (int g = j; g < gcount; g += 32)
                    v += ps[g];
            }
#pragma unroll
            for (int off = 16; off >= 1; off >>= 1)
                v += __shfl_xor(v, off, 32);
            if (row_live && j == 0) {
                float t = acc_tile[m][r] + v;
                acc_tile[m][r] = t;
                if (last) {
                    int n = n0 + r;
                    if (a.yt == VBQ_F16)
                        reinterpret_cast<__half *>(a.y)[(uint64_t)m * a.ldy + n] = __float2half_rn(t);
                    else
                        reinterpret_cast<float *>(a.y)[(uint64_t)m * a.ldy + n] = t;
                }
            }
        }
        u = nu;
    }
}

int tokens_template(int M) { return M <= 1 ? 1 : M <= 2 ? 2 : M <= 4 ? 4 : M <= 8 ? 8 : 16; }

struct Plan {
    int R, SG, CHK, slots, tiles;
    size_t smem;
};

Plan make_plan(const vbq_layout *L, int MT)
{
    Plan p;
    int nS = (int)L->nS;
    p.CHK = std::min(nS, std::max(1, 16 / MT));       // x image <= 64 KiB
    p.slots = MT <= 2 ? 1024 : MT == 4 ? 512 : 256;   // slot-table capacity
    // tall tiles when there are enough rows to keep every CU busy
    int R = 32;
    while (R > 8 && ((int64_t)L->N + R - 1) / R < 1024)
        R /= 2;
    R = std::min(R, p.slots / 32);
    p.R = std::max(1, R);
    p.SG = std::max(1, std::min(p.CHK, std::min(p.slots / (32 * p.R), kMaxRS / p.R)));
    p.tiles = (int)(((int64_t)L->N + p.R - 1) / p.R);
    size_t chg = (size_t)p.CHK * 32;
    p.smem = (size_t)MT * chg * 32 * 4 + (size_t)MT * chg * 4 * 4 + (size_t)p.slots * 8 +
             (size_t)MT * p.R * (p.SG * 32 + 1) * 4;
    return p;
}

template <int MT>
vbq_status launch(GemvArgs a, const Plan &p, hipStream_t stream)
{
    VBQ_TRY(dynamic_lds_once((const void *)k_gemv<MT>, 96 * 1024));
    const int cus = current_device_cus();
    int per_cu = 0;
    VBQ_TRY(hip_status(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)k_gemv<MT>, kThreads,
                                                                     p.smem)));
    if (per_cu < 1)
        return VBQ_ERR_SHAPE;
    int grid = std::min(p.tiles, per_cu * cus);
    a.R = p.R;
    a.SG = p.SG;
    a.CHK = p.CHK;
    a.tiles = p.tiles;
    a.slots = p.slots;
    hipLaunchKernelGGL(k_gemv<MT>, dim3(grid), dim3(kThreads), p.smem, stream, a);
    return launch_status();
}




} // namespace

extern "C" {

vbq_status vbq_workspace_size(const vbq_layout *L, int M, size_t *bytes)
{
    if (!bytes)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if (M < 1 || M > kMaxBatch)
        return VBQ_ERR_BATCH;
    // the matrix cores take 3 or more tokens, and fewer where the streaming
    // kernel does not apply
    *bytes = M >= kMfmaMinTokens || !stream_applies(L, M) ? mfma_workspace(L, M) : 0;
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
    if (M < 1 || M > kMaxBatch)
        return VBQ_ERR_BATCH;
    if (ldx < (int)L->K || ldy < (int)L->N)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)blob % 256 || (uintptr_t)x % 2 || (uintptr_t)y % (yt == VBQ_F32 ? 4 : 2))
        return VBQ_ERR_ALIGN;
    {
        GemvCall call{L, blob, M, x, ldx, y, ldy, yt, stream};
        const bool mfma = mfma_applies(L, M, x, ldx);
        if (mfma && M >= kMfmaMinTokens)
            return mfma_gemv(call, ws, ws_bytes);
        if (M > 16) // only the matrix cores take more than 16 tokens
            return (uintptr_t)x % 16 || ldx % 8 ? VBQ_ERR_ALIGN : VBQ_ERR_SHAPE;
        vbq_status st;
        if (stream_gemv(call, &st))
            return st;
        // one or two tokens on a matrix the streaming kernel does not take
        // (K > 16256): the matrix cores, which unpack each code once all the same
        if (mfma)
            return mfma_gemv(call, ws, ws_bytes);
    }
    const int MT = tokens_template(M);
    Plan p = make_plan(L, MT);
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
    switch (MT) {
    case 1: return launch<1>(a, p, stream);
    case 2: return launch<2>(a, p, stream);
    case 4: return launch<4>(a, p, stream);
    case 8: return launch<8>(a, p, stream);
    default: return launch<16>(a, p, stream);
    }
}

vbq_status vbq_gemv_shared(const vbq_gemv_item *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                           hipStream_t stream)
{
    if (!items || n < 1 || n > VBQ_MAX_SHARED || !x)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    StreamItem st_items[VBQ_MAX_SHARED];
    for (int i = 0; i < n; i++) {
        const vbq_gemv_item &it = items[i];
        if (!it.L || !it.blob || !it.y)
            return VBQ_ERR_INVALID_ARG;
        VBQ_TRY(check_layout(it.L));
        if (it.L->K != items[0].L->K || ldx < (int)it.L->K || it.ldy < (int)it.L->N)
            return VBQ_ERR_SHAPE;
        if ((uintptr_t)it.blob % 256 || (uintptr_t)it.y % (yt == VBQ_F32 ? 4 : 2))
            return VBQ_ERR_ALIGN;
        st_items[i] = StreamItem{it.L, it.blob, it.y, it.ldy};
    }
    if ((uintptr_t)x % 2)
        return VBQ_ERR_ALIGN;
    vbq_status st;
    if (stream_gemv_shared(st_items, n, M, x, ldx, yt, stream, &st))
        return st;
    for (int i = 0; i < n; i++) // one launch per matrix where the streaming kernel does not apply
        VBQ_TRY(vbq_gemv_batched(items[i].L, items[i].blob, M, x, ldx, items[i].y, items[i].ldy, yt, nullptr, 0,
                                 stream));
    return VBQ_OK;
}

vbq_status vbq_gemv(const vbq_layout *L, const void *blob, const uint16_t *x, void *y, vbq_dtype yt, void *ws,
                    size_t ws_bytes, hipStream_t stream)
{
    if (!L)
        return VBQ_ERR_INVALID_ARG;
    return vbq_gemv_batched(L, blob, 1, x, (int)L->K, y, (int)L->N, yt, ws, ws_bytes, stream);
}

} // extern "C"
