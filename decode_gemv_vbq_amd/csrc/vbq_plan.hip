// Prepared GEMV plans: a one-time device re-encoding of a VBQ1 matrix into
// the order in which the decode kernel consumes it, and that kernel.
//
// The method ("Variable Bit-width Quantization", mlsanity.com page, Abstract)
// gives every contiguous group of 64 weights its own width in {1,2,4,8}, and
// decode, which is bound by memory bandwidth, multiplies the packed codes
// without materialising the weights.  A wavefront must run groups of ONE
// width at a time; the VBQ1 blob stores groups row by row, so a kernel that
// reads it directly has to sort every tile by width at run time.  A plan does
// that sort once per matrix, and lays the result out so that the GEMV never
// waits for metadata before it can fetch weights:
//
//  * The rows are split into row blocks, one per workgroup of the GEMV
//    launch; block b owns a region of the plan buffer at a fixed stride.
//  * A block's groups are sorted by (width 1,2,4,8; column; row) and cut into
//    PASSES of 1 KiB of codes: 128 one-bit groups, 64 two-bit, 32 four-bit or
//    16 eight-bit groups.  Every pass record has the same size (1536 bytes:
//    the codes, then one 32-bit word per group: fp16 scale | position << 16,
//    position = column * stride + row), so the address of pass p is
//    region + 1536 p and a wavefront can issue its loads before it knows
//    anything else about the pass.
//  * After the passes, one byte per pass gives its width (0: no pass), laid
//    out wave-major for the 16 wavefronts of the GEMV workgroup.
//
// The GEMV kernel: one 1024-thread workgroup per row block; wavefront w takes
// passes w, w+16, w+32, ... and keeps the next two of them in flight from
// HBM straight into registers while it computes one (16 bytes of codes and 8
// bytes of words per lane, the same two loads for every width).  Lane l holds
// groups 2l and 2l+1 of a one-bit pass, group l of a two-bit pass, half of
// group l/2 of a four-bit pass, a quarter of group l/4 of an eight-bit pass.
// The activations are staged once per workgroup as records of fp16 pairs
// (x_p, x_{p+32}) and per-width corrections; each group's dot products land
// as one fp32 partial at its position in LDS.  Two barriers per launch (the
// records are ready; every partial is written), then the rows are summed in
// a fixed order, so the result does not depend on timing.
#include <algorithm>
#include <type_traits>

#include "vbq_common.h"
#include "vbq_host.h"
#include "vbq_unpack.h"

using namespace vbq;

namespace {

constexpr int kT = 1024; // threads per workgroup (prepare and GEMV kernels)
constexpr int kW = kT / 64;
constexpr int kPassBytes = 1536; // one pass record
constexpr int kCodeArea = 1024;  // its code bytes: 16 per lane
constexpr int kXRec = 36;        // dwords of x per group: 32 pairs (x_p, x_{p+32}) + 4 constants
constexpr int kMaxG = 512;       // groups per row the plans support (K <= 32768)
constexpr int kMaxPerWave = 256; // width bytes per wavefront (passes <= 16 * 255)
constexpr int kMaxMats = VBQ_MAX_SHARED;
constexpr uint32_t kLdsBudget = 160u * 1024u;

__host__ __device__ constexpr int groups_per_pass(int c) { return 128 >> c; } // c = log2(width)

// Width bytes per wavefront for a region of `passes` pass records (every
// wavefront's list ends with a 0; a multiple of 4), and the region's bytes.
__host__ __device__ constexpr int per_wave_for(int passes) { return ((passes + kW - 1) / kW + 1 + 3) & ~3; }
__host__ __device__ constexpr uint32_t region_for(int passes, int per_wave)
{
    return ((uint32_t)passes * kPassBytes + (uint32_t)kW * per_wave + 255u) & ~255u;
}

// Position stride of a block: position = column * stride + row.  At least 2,
// so that the column is always a 32-bit reciprocal multiply away.  From 32
// rows on it is padded to 64 / L modulo 32 (L lanes sum a row at the end, L
// by G as in sum_lanes), so that the L lanes of a row and the 64 / L rows of a
// wavefront read the partial sums from distinct LDS banks (two lanes per bank,
// the least for 64 lanes): 2% on a 9B decode step.
__host__ __device__ constexpr int sum_lanes_of(int G) { return G > 256 ? 64 : G > 128 ? 32 : G > 64 ? 16 : 8; }
__host__ __device__ constexpr int pos_stride(int rows, int G)
{
    const int r = rows < 2 ? 2 : rows, want = 64 / sum_lanes_of(G);
    return r < 32 ? r : r + ((want - r) % 32 + 32) % 32;
}

// Partial sums per token in LDS: every position of the widest block plus one
// slot that the empty places of a partly filled pass write to.
__host__ __device__ constexpr int psum_stride(int G, int stride) { return (stride * G + 1 + 3) & ~3; }

// ---------------------------------------------------------------------------
// Block-wide exclusive scan of one value per thread (kT threads).
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t *tmp /* LDS, kW + 1 */, uint32_t &total)
{
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d);
        if (lane >= d)
            inc += o;
    }
    if (lane == 63)
        tmp[wave] = inc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t run = 0;
        for (int w = 0; w < kW; w++) {
            const uint32_t t = tmp[w];
            tmp[w] = run;
            run += t;
        }
        tmp[kW] = run;
    }
    __syncthreads();
    const uint32_t ex = tmp[wave] + inc - v;
    total = tmp[kW];
    __syncthreads(); // tmp is reused by the next call
    return ex;
}

// Width code (log2 b) of group (row n of the matrix, column g) from the VBQ1 bit planes.
__device__ __forceinline__ int vbq1_width(const uint32_t *wmap, int nS, int n, int g)
{
    const uint64_t rs = (uint64_t)n * nS + (g >> 5);
    return width_code(wmap[2 * rs], wmap[2 * rs + 1], g & 31);
}

struct PrepArgs {
    const uint8_t *blob;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    int N, G, nS, rows;
    int passes;       // pass records per block region (fill)
    int per_wave;     // width bytes per wavefront (fill)
    uint64_t region;  // bytes per block region
    uint8_t *plan;    // null: sizing only
    uint32_t *sizes;  // sizing: [0] the largest block's pass count
    uint32_t *status; // fill (may be null): VBQ_STATUS_PLAN when a block needs more passes than `passes`
};

// One workgroup per row block.  Groups are counted per (width, column); an
// exclusive scan in (width 1,2,4,8; column) order gives each bucket its first
// slot, and inside a bucket the rows follow in order.  Slot s of width c is
// group s % groups_per_pass(c) of pass P_c + s / groups_per_pass(c), where
// the passes of the narrower widths come first.
__global__ __launch_bounds__(kT) void k_prepare(PrepArgs a)
{
    __shared__ uint32_t tmp[kW + 1];
    __shared__ uint32_t hist[4 * kMaxG]; // per (width, column): count, then first slot
    const int tid = threadIdx.x;
    const int n0 = (int)blockIdx.x * a.rows;
    if (n0 >= a.N)
        return;
    const int R = min(a.rows, a.N - n0);
    const int G = a.G;
    const uint32_t NG = (uint32_t)R * (uint32_t)G;
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
    for (int k = tid; k < 4 * G; k += kT)
        hist[k] = 0;
    __syncthreads();
    for (uint32_t i = (uint32_t)tid; i < NG; i += kT) {
        const int r = (int)(i / (uint32_t)G), g = (int)(i - (uint32_t)r * G);
        atomicAdd(&hist[vbq1_width(wmap, a.nS, n0 + r, g) * G + g], 1u);
    }
    __syncthreads();
    {
        uint32_t carry = 0;
        for (int base = 0; base < 4 * G; base += kT) {
            const int k = base + tid;
            const uint32_t v = k < 4 * G ? hist[k] : 0u;
            uint32_t tot;
            const uint32_t ex = block_excl_scan(v, tmp, tot);
            if (k < 4 * G)
                hist[k] = carry + ex;
            carry += tot;
            __syncthreads();
        }
    }
    uint32_t S[5], P0[5]; // first slot and first pass of each width
    for (int c = 0; c < 4; c++)
        S[c] = hist[c * G];
    S[4] = NG;
    P0[0] = 0;
    for (int c = 0; c < 4; c++)
        P0[c + 1] = P0[c] + (S[c + 1] - S[c] + groups_per_pass(c) - 1) / groups_per_pass(c);
    const uint32_t npass = P0[4];
    if (!a.plan) {
        if (tid == 0)
            atomicMax(a.sizes, npass);
        return;
    }
    if (npass > (uint32_t)a.passes) { // the plan was sized for other widths: write nothing
        if (tid == 0 && a.status)
            atomicOr(a.status, VBQ_STATUS_PLAN);
        return;
    }
    uint8_t *region = a.plan + (uint64_t)blockIdx.x * a.region;
    const int stride = pos_stride(a.rows, a.G);
    const uint32_t dummy = (uint32_t)(stride * G) << 16; // scale 0 at the spare position
    // Word area of a pass of width code c: group k's word at the 2^c u32 slots
    // k 2^c .. (k + 1) 2^c - 1, so that the 8 bytes lane l loads (slots 2l,
    // 2l + 1) hold the words of the groups lane l works on: groups 2l, 2l + 1
    // of a one-bit pass, the one group of the lane otherwise (the 512 bytes
    // are full for every width).
    // the empty places of each width's last pass: zero codes, the spare position
    for (int c = 0; c < 4; c++) {
        const int per = groups_per_pass(c);
        const int used = (int)((S[c + 1] - S[c]) % (uint32_t)per);
        if (!used)
            continue;
        uint8_t *rec = region + (uint64_t)(P0[c + 1] - 1) * kPassBytes;
        for (int k = used + tid; k < per; k += kT) {
            uint32_t *d32 = reinterpret_cast<uint32_t *>(rec + k * (8 << c));
            for (int d = 0; d < (2 << c); d++)
                d32[d] = 0u;
            for (int d = 0; d < (1 << c); d++)
                reinterpret_cast<uint32_t *>(rec + kCodeArea)[(k << c) + d] = dummy;
        }
    }
    // the groups: thread g walks column g's rows, so each bucket's rows follow in order
    const uint32_t *rowoff = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off);
    const uint32_t *sloff = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.blob + a.off_scales);
    const uint8_t *codes = a.blob + a.off_codes;
    for (int g = tid; g < G; g += kT) {
        uint32_t run[4] = {0, 0, 0, 0};
        for (int r = 0; r < R; r++) {
            const int nn = n0 + r;
            const uint64_t rs = (uint64_t)nn * a.nS + (g >> 5);
            const uint32_t p0 = wmap[2 * rs], p1 = wmap[2 * rs + 1];
            const WidthMasks wm = width_masks(p0, p1, min(32, G - 32 * (g >> 5)));
            const int c = width_code(p0, p1, g & 31);
            const uint32_t s = hist[c * G + g] - pick4(S, c) + pick4(run, c);
            run[0] += c == 0;
            run[1] += c == 1;
            run[2] += c == 2;
            run[3] += c == 3;
            const uint32_t per = (uint32_t)groups_per_pass(c);
            uint8_t *rec = region + (uint64_t)(pick4(P0, c) + s / per) * kPassBytes;
            const uint32_t k = s % per;
            const uint64_t src = (uint64_t)rowoff[nn] * kRowPad + sloff[rs] + group_offset_in_slice(wm, c, g & 31);
            const uint32_t *s32 = reinterpret_cast<const uint32_t *>(codes + src);
            uint32_t *d32 = reinterpret_cast<uint32_t *>(rec + k * (8u << c));
            for (int d = 0; d < (2 << c); d++)
                d32[d] = s32[d];
            const uint32_t e = (uint32_t)g * (uint32_t)stride + (uint32_t)r;
            const uint32_t word = (uint32_t)scales[(uint64_t)nn * G + g] | (e << 16);
            for (int d = 0; d < (1 << c); d++)
                reinterpret_cast<uint32_t *>(rec + kCodeArea)[(k << c) + d] = word;
        }
    }
    // width bytes, wave-major: pass w + 16 j at byte w * per_wave + j
    uint8_t *meta = region + (uint64_t)a.passes * kPassBytes;
    for (int i = tid; i < kW * a.per_wave; i += kT) {
        const int w = i / a.per_wave, j = i - w * a.per_wave;
        const uint32_t p = (uint32_t)(w + kW * j);
        uint8_t v = 0;
        if (p < npass)
            v = (uint8_t)(1 + (p >= P0[1]) + (p >= P0[2]) + (p >= P0[3]));
        meta[i] = v;
    }
}

// ---------------------------------------------------------------------------
// The planned GEMV kernel.

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// 64 bytes of the kernel-argument segment at byte offset `off` (a multiple of
// 64) in one scalar load; the wait is inside the asm block, so no load is
// left in flight when it ends.
__device__ __forceinline__ u32x16 kernarg_line(uint32_t off)
{
    u32x16 r;
    asm volatile("s_load_dwordx16 %0, %1, %2\n\ts_waitcnt lgkmcnt(0)"
                 : "=s"(r)
                 : "s"(__builtin_amdgcn_kernarg_segment_ptr()), "s"(off)
                 : "memory");
    return r;
}

__device__ __forceinline__ const void *u64_ptr(uint32_t lo, uint32_t hi)
{
    return (const void *)(((uint64_t)hi << 32) | lo);
}

// Kernel arguments.  The argument segment is read from memory at every
// launch and is not kept in the caches between launches, so each round of
// dependent argument loads costs a full memory round trip before a workgroup
// can start.  A workgroup therefore finds everything it needs in ONE 64-byte
// record, picked by blockIdx.y (the matrix of a shared launch), which it reads
// with a single scalar load.  Launch-wide fields are repeated in every record.
struct PRec {
    const uint8_t *plan; // this matrix's plan
    void *y;             // its outputs (this launch's first token)
    const uint16_t *x;   // activations (this launch's first token)
    uint32_t region;     // bytes per row block of the plan
    int32_t N, ldy, rows; // rows per block of this matrix
    int32_t ldx;
    int32_t passes;      // pass records per block region
    int32_t per_wave;    // width bytes per wavefront
    uint32_t g_yt;       // G | yt << 16 (launch-wide)
    int32_t wgs;         // row blocks of this matrix (workgroups with blockIdx.x < wgs work)
    int32_t smax;        // largest position stride of the launch's plans (LDS carve-up)
};
static_assert(sizeof(PRec) == 64, "one record is one 64-byte line");

struct PArgs {
    PRec rec[kMaxMats];
};

struct PLayout {
    uint32_t x, psum, ybuf, best, total;
};

__host__ __device__ inline uint32_t p_take(uint32_t &o, uint32_t bytes)
{
    const uint32_t r = o;
    o += (bytes + 15u) & ~15u;
    return r;
}

// LDS carve-up, computed identically on the host (size) and the device.  One
// x record more than the tokens need: the spare position of a partly filled
// pass decodes to column G and reads it (its result is never used).
__host__ __device__ inline PLayout p_layout(int MT, int G, int smax)
{
    PLayout l;
    uint32_t o = 0;
    l.x = p_take(o, (uint32_t)((MT * G + 1) * kXRec * 4));
    l.psum = p_take(o, (uint32_t)(MT * psum_stride(G, smax)) * 4u);
    l.ybuf = p_take(o, (uint32_t)(MT * smax) * 4u);
    l.best = p_take(o, 2u * 8u); // argmax output: the best (value, row) key per token
    l.total = o;
    return l;
}

// x records (kXRec dwords per group; the 36-dword stride spreads the records
// of different columns over the LDS banks): the fp16 pairs (x_p, x_{p+32}),
// then the negated corrections -C_b for the widths 1, 2, 4, 8, where
// C_b = sum_p 2^(10-pos_b(p)) (x_p + x_{p+32}) + (2^b-1)/2 sum_j x_j.
// Item = (token, group, part r): pairs 8r..8r+7, from one 16-byte load of
// x_{8r..8r+7} and one of x_{32+8r..32+8r+7}; the 4 items of a group are 4
// adjacent lanes.  Loads and stores are separate so that the loads go out
// before the first passes' loads and the wait for them leaves those in flight.
// KP items per thread: MT * G * 4 items rounded up to a power of two over the
// workgroup (chosen per launch, so that no more loads are issued than needed).
// Sum of v over each aligned group of 4 lanes, the same value in every lane of
// the group, in a fixed order: pairs, then the two pairs (DPP quad permutations).
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_f<0xB1>(v); // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v); // quad_perm [2, 3, 0, 1]
    return v;
}

template <int KP>
struct XRegs {
    static constexpr int kPer = KP;
    u32x4 lo[KP], hi[KP];
};

template <int MT, int KP>
__device__ __forceinline__ void x_load(const uint16_t *x, int ldx, int G, XRegs<KP> &xs)
{
    static_assert(MT <= 2, "the planned path takes one or two tokens");
    // x is 8-byte aligned and ldx a multiple of 4 (checked on the host): two
    // 16-byte buffer loads per item (dword-aligned, as buffer loads need).
    // Every load is issued (so that the wait for them is exact), and a
    // compiler barrier keeps them ahead of the pass loads, so that this wait
    // leaves those in flight.
    const int tid = threadIdx.x;
    const int items = MT * G * 4;
    const int nrec = (int)(((MT - 1) * (uint32_t)ldx + 64u * (uint32_t)G) * 2u); // < 2^31: checked on the host
    const __amdgpu_buffer_rsrc_t xr = __builtin_amdgcn_make_buffer_rsrc((void *)x, 0, nrec, 0x00020000);
#pragma unroll
    for (int k = 0; k < KP; k++) {
        const int i = tid + k * kT;
        // item i: token m, group g, part r (at most two tokens: a compare,
        // not a division by G, which would delay the loads)
        const int r = i & 3, m = (MT > 1 && (i >> 2) >= G) ? 1 : 0, g = (i >> 2) - m * G;
        // a lane past the last item gets an offset past the buffer: the load
        // returns zeros without a memory access
        const int off = i < items ? (m * ldx + 64 * g + 8 * r) * 2 : nrec;
        xs.lo[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0);
        xs.hi[k] = __builtin_amdgcn_raw_buffer_load_b128(xr, off + 64, 0, 0);
    }
    asm volatile("" ::: "memory");
}

template <int MT, int KP>
__device__ __forceinline__ void x_store(int G, const XRegs<KP> &xs, uint32_t *xrec)
{
    const int tid = threadIdx.x;
    const int items = MT * G * 4;
#pragma unroll
    for (int k = 0; k < KP; k++) {
        const int i = tid + k * kT;
        if (i >= items) // whole groups of 4 lanes drop out together
            break;
        const int r = i & 3, m = (MT > 1 && (i >> 2) >= G) ? 1 : 0, g = (i >> 2) - m * G;
        uint32_t pr[8];
#pragma unroll
        for (int h = 0; h < 4; h++) {
            pr[2 * h] = __builtin_amdgcn_perm(xs.hi[k][h], xs.lo[k][h], 0x05040100u);     // (x_p, x_{p+32})
            pr[2 * h + 1] = __builtin_amdgcn_perm(xs.hi[k][h], xs.lo[k][h], 0x07060302u); // next p
        }
        uint32_t *xr = xrec + ((uint32_t)m * G + g) * kXRec;
        *reinterpret_cast<U4 *>(xr + 8 * r) = U4{{pr[0], pr[1], pr[2], pr[3]}};
        *reinterpret_cast<U4 *>(xr + 8 * r + 4) = U4{{pr[4], pr[5], pr[6], pr[7]}};
        float X = 0.f, c1 = 0.f, c2 = 0.f, c4 = 0.f;
#pragma unroll
        for (int j = 0; j < 8; j++) {
            const int t = 8 * r + j; // pair index in the group
            const float sp = dot2(pr[j], 0x3c003c00u, 0.f); // x_t + x_{t+32}, exact in fp32
            X += sp;
            c1 = fmaf((float)(1 << (10 - pair_pos<1>(t & 15))), sp, c1);
            c2 = fmaf((float)(1 << (10 - pair_pos<2>(t & 7))), sp, c2);
            c4 = fmaf((float)(1 << (10 - pair_pos<4>(t & 3))), sp, c4);
        }
        // fixed-order tree over the 4 parts of the group
        X = quad_sum(X);
        c1 = quad_sum(c1);
        c2 = quad_sum(c2);
        c4 = quad_sum(c4);
        if (r == 0)
            *reinterpret_cast<U4 *>(xr + 32) =
                U4{{__float_as_uint(-fmaf(0.5f, X, c1)), __float_as_uint(-fmaf(1.5f, X, c2)),
                    __float_as_uint(-fmaf(7.5f, X, c4)), __float_as_uint(-fmaf(127.5f, X, 1024.f * X))}};
    }
}

// One pass in flight: this lane's 16 code bytes and 8 word bytes.
struct PBuf {
    u32x4 c;
    u32x2 w;
};

// What the pass bodies share.
struct PCtx {
    const uint32_t *xrec;
    float *psum;
    int G, ps;
    uint32_t inv; // ceil(2^32 / stride): column = umulhi(position, inv)
};

// Dot products of NP pairs of one group (its pairs p0 .. p0 + NP - 1) with
// every token's x record of column `col`: one fp32 chain, starting
// from the group's -C_b when this lane carries the correction.
template <int C, int NP, int MT>
__device__ __forceinline__ void dot_pairs(const uint32_t *hp, int p0, bool corr, uint32_t col, const PCtx &cx,
                                          float *acc)
{
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const uint32_t *xr = cx.xrec + ((uint32_t)m * cx.G + col) * kXRec;
        const float c0 = __uint_as_float(xr[32 + C]);
        float a = corr ? c0 : 0.f;
#pragma unroll
        for (int k = 0; k < NP / 4; k++) {
            const U4 xa = *reinterpret_cast<const U4 *>(xr + p0 + 4 * k);
#pragma unroll
            for (int t = 0; t < 4; t++)
                a = dot2(hp[4 * k + t], xa.v[t], a);
        }
        acc[m] = a;
    }
}

__device__ __forceinline__ float scale_of(uint32_t se) { return __half2float(__ushort_as_half((uint16_t)(se & 0xffffu))); }

// s * v for the fp16 scale s in the low half of se.  (A hand-written
// mixed-precision fma saves the conversion, but the compiler does not insert
// the wait states a VALU read of a v_dot2c result needs when the reader is
// inline asm, so it read a stale sum on gfx950.)
__device__ __forceinline__ float scaled(uint32_t se, float v) { return scale_of(se) * v; }

// One-bit pass: this lane's groups 2l and 2l+1 (8 code bytes and one word each).
template <int MT>
__device__ __forceinline__ void pass_b1(const PBuf &b, const PCtx &cx)
{
#pragma unroll
    for (int h = 0; h < 2; h++) {
        const uint32_t w[2] = {b.c[2 * h], b.c[2 * h + 1]};
        uint32_t hp[32];
        unpack_pairs<1>(w, hp);
        const uint32_t se = b.w[h], e = se >> 16;
        float acc[MT];
        dot_pairs<0, 32, MT>(hp, 0, true, __umulhi(e, cx.inv), cx, acc);
#pragma unroll
        for (int m = 0; m < MT; m++)
            cx.psum[m * cx.ps + e] = scaled(se, acc[m]);
    }
}

// Two-bit pass: group l (16 code bytes; its word is the first of the lane's
// two word-area slots, as for the four- and eight-bit passes).
template <int MT>
__device__ __forceinline__ void pass_b2(const PBuf &b, const PCtx &cx)
{
    const uint32_t se = b.w[0], e = se >> 16;
    const uint32_t w[4] = {b.c[0], b.c[1], b.c[2], b.c[3]};
    uint32_t hp[32];
    unpack_pairs<2>(w, hp);
    float acc[MT];
    dot_pairs<1, 32, MT>(hp, 0, true, __umulhi(e, cx.inv), cx, acc);
#pragma unroll
    for (int m = 0; m < MT; m++)
        cx.psum[m * cx.ps + e] = scaled(se, acc[m]);
}

// Four-bit pass: half h = l & 1 of group l >> 1 (its words 4h..4h+3, pairs
// 16h..16h+15); the two lanes' sums are added, the even lane writes.
template <int MT>
__device__ __forceinline__ void pass_b4(const PBuf &b, const PCtx &cx)
{
    const int lane = threadIdx.x & 63, h = lane & 1;
    const uint32_t se = b.w[0], e = se >> 16;
    const uint32_t w[4] = {b.c[0], b.c[1], b.c[2], b.c[3]};
    uint32_t hp[16];
    unpack_words<4, 4>(w, hp);
    float acc[MT];
    dot_pairs<2, 16, MT>(hp, 16 * h, h == 0, __umulhi(e, cx.inv), cx, acc);
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const float v = acc[m] + dpp_f<0xB1>(acc[m]); // quad_perm [1, 0, 3, 2]
        if (h == 0)
            cx.psum[m * cx.ps + e] = scaled(se, v);
    }
}

// Eight-bit pass: quarter q = l & 3 of group l >> 2 (its words 4q..4q+3,
// pairs 8q..8q+7); the four lanes' sums are added in a fixed order, the first
// lane writes.
template <int MT>
__device__ __forceinline__ void pass_b8(const PBuf &b, const PCtx &cx)
{
    const int lane = threadIdx.x & 63, q = lane & 3;
    const uint32_t se = b.w[0], e = se >> 16;
    const uint32_t w[4] = {b.c[0], b.c[1], b.c[2], b.c[3]};
    uint32_t hp[8];
    unpack_words<8, 4>(w, hp);
    float acc[MT];
    dot_pairs<3, 8, MT>(hp, 8 * q, q == 0, __umulhi(e, cx.inv), cx, acc);
#pragma unroll
    for (int m = 0; m < MT; m++) {
        float v = acc[m] + dpp_f<0xB1>(acc[m]); // quad_perm [1, 0, 3, 2]
        v += dpp_f<0x4E>(v);                    // quad_perm [2, 3, 0, 1]
        if (q == 0)
            cx.psum[m * cx.ps + e] = scaled(se, v);
    }
}

// Lanes that sum one row: more for longer rows, so that the row sums stay
// short (a row of G partials is G / lanes loads deep).
__device__ __forceinline__ int sum_lanes(int G) { return sum_lanes_of(G); }

// Output modes, a template parameter of the kernel (a plain GEMV carries no
// code of the others).  kRows: finished rows are stored as fp32 or fp16 (yt).
// kArgmax: instead of storing rows, keep per token the largest (value,
// smallest row) as one 64-bit key in LDS (see argmax_key).  kSwiglu: rows 2i
// and 2i+1 are the gate and up rows of output i; row sums stay in LDS and the
// workgroup writes silu(gate) * up (type yt) for its pairs at the end.
constexpr int kRows = 0;
constexpr int kArgmax = 1;
constexpr int kSwiglu = 2;

// Outputs are stored through global (address space 1) pointers: a store
// through a generic pointer is a flat store, which also counts on the counter
// the LDS reads of the row sums wait on, so that every wait for them would
// also wait for the previous row's store.
typedef __attribute__((address_space(1))) uint16_t gu16_t;
typedef __attribute__((address_space(1))) float gf32_t;

struct YOut {
    void *y;
    int ldy, n0, yt, smax;
    unsigned long long *best; // LDS, [MT] keys (kArgmax)
};

// Order-preserving key of (value, row): the fp32 bits mapped so that unsigned
// order is the IEEE total order (-NaN < -inf < ... < +inf < +NaN), then the
// complemented row, so that the maximum key is the largest value at its
// smallest row.
__device__ __forceinline__ unsigned long long argmax_key(float v, uint32_t row)
{
    const uint32_t u = __float_as_uint(v);
    const uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((unsigned long long)ord << 32) | (unsigned long long)(~row);
}

// Sum of the C partials of one row that one lane adds (pg: the first, step:
// the distance to the next), all loaded at once, in the order of the general
// loop below: four chains over whole rounds of four columns, the remaining
// columns into the first chain, then (chain 0 + chain 1) + (chain 2 + chain 3).
template <int C>
__device__ __forceinline__ float cols_sum(const float *pg, int step)
{
    float x[C];
#pragma unroll
    for (int k = 0; k < C; k++)
        x[k] = pg[k * step];
    float a[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < C / 4 * 4; k++)
        a[k & 3] += x[k];
#pragma unroll
    for (int k = C / 4 * 4; k < C; k++)
        a[0] += x[k];
    return (a[0] + a[1]) + (a[2] + a[3]);
}

// Row sums of the block, L lanes per row.  Item t (t = wave, wave + kW, ...)
// covers rows (64 / L) t .. of the block.  The partials of row j sit at
// column * stride + j; lane q adds its columns q, q + L, ... in four chains
// (cols_sum: whole rounds of four first, the rest into the first chain) and
// the L lanes of the row combine in a fixed order (group_sum).  C > 0: every
// lane has C columns (G = C * L), a straight run of loads and adds; C = 0: any
// G, the same additions as loops.  Both give the same bits for a row.
template <int MT, int OM, int L, int C>
__device__ __forceinline__ void row_sums_lc(int wave, int R, int stride, int G, int ps, const float *psum,
                                            float *ybuf, const YOut &yo)
{
    constexpr int per = 64 / L;
    const int lane = threadIdx.x & 63;
    const int q = lane & (L - 1);
    const int nsum = (R * L + 63) / 64;
    const int step = L * stride; // column g + L of the row sits L * stride further
    for (int t = wave; t < nsum; t += kW) {
        const int j = per * t + lane / L;
#pragma unroll
        for (int m = 0; m < MT; m++) {
            float v = 0.f;
            if constexpr (C > 0) {
                // a lane past the last row sums row R - 1 again (not stored)
                v = cols_sum<C>(psum + m * ps + min(j, R - 1) + q * stride, step);
            } else if (j < R) {
                const float *pg = psum + m * ps + j + q * stride;
                float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
                int g = q;
                for (; g + 3 * L < G; g += 4 * L, pg += 4 * step) {
                    a0 += pg[0];
                    a1 += pg[step];
                    a2 += pg[2 * step];
                    a3 += pg[3 * step];
                }
                for (; g < G; g += L, pg += step)
                    a0 += pg[0];
                v = (a0 + a1) + (a2 + a3);
            }
            v = group_sum<L>(v);
            if (q == 0 && j < R) {
                const uint64_t o = (uint64_t)m * yo.ldy + yo.n0 + j;
                if constexpr (OM == kArgmax)
                    atomicMax(yo.best + m, argmax_key(v, (uint32_t)(yo.n0 + j)));
                else if constexpr (OM == kSwiglu)
                    ybuf[m * yo.smax + j] = v;
                else if (yo.yt == VBQ_F16)
                    ((gu16_t *)yo.y)[o] = __half_as_ushort(__float2half_rn(v));
                else
                    ((gf32_t *)yo.y)[o] = v;
            }
        }
    }
}

// Row shape of a launch as one number, L * 16 + C: L lanes per row (by G) and
// C columns per lane when every lane has the same number and it is 4, 7 or 8
// (G = 4L, 7L or 8L: every decode shape of the 1B and 9B steps), else C = 0.
// (Four columns per lane only occur at L = 8: from G = 65 on, L >= 16 and
// G / L > 4.)
__host__ __device__ constexpr int row_shape_of(int G)
{
    const int L = sum_lanes_of(G), c = G / L;
    return L * 16 + ((c * L == G && (c == 4 || c == 7 || c == 8)) ? c : 0);
}

// The row-sum code of a launch.  A launch ends shortly after it, and every
// wavefront of the last workgroups runs it at once, so what it executes there
// (scalar work included) is on the launch's critical path.  RS > 0: the row
// shape is a template argument (the launches with preloaded arguments; the
// host picks the kernel); RS = 0: chosen by G at run time.  Measured on a 9B
// decode step: the straight run for G = 8L chosen by the host against one
// general loop chosen per item, -3.5%.
template <int MT, int OM, int RS>
__device__ __forceinline__ void row_sums(int wave, int R, int stride, int G, int ps, const float *psum, float *ybuf,
                                         const YOut &yo)
{
#define VBQ_ROWS(S_) row_sums_lc<MT, OM, (S_) / 16, (S_) % 16>(wave, R, stride, G, ps, psum, ybuf, yo)
    if constexpr (RS > 0) {
        VBQ_ROWS(RS);
    } else {
        switch (row_shape_of(G)) {
        case 8 * 16 + 8: VBQ_ROWS(8 * 16 + 8); break;
        case 8 * 16 + 7: VBQ_ROWS(8 * 16 + 7); break;
        case 8 * 16 + 4: VBQ_ROWS(8 * 16 + 4); break;
        case 8 * 16: VBQ_ROWS(8 * 16); break;
        case 16 * 16 + 8: VBQ_ROWS(16 * 16 + 8); break;
        case 16 * 16 + 7: VBQ_ROWS(16 * 16 + 7); break;
        case 16 * 16: VBQ_ROWS(16 * 16); break;
        case 32 * 16 + 8: VBQ_ROWS(32 * 16 + 8); break;
        case 32 * 16 + 7: VBQ_ROWS(32 * 16 + 7); break;
        case 32 * 16: VBQ_ROWS(32 * 16); break;
        case 64 * 16 + 8: VBQ_ROWS(64 * 16 + 8); break;
        case 64 * 16 + 7: VBQ_ROWS(64 * 16 + 7); break;
        default: VBQ_ROWS(64 * 16); break;
        }
    }
#undef VBQ_ROWS
}

// Merge this workgroup's keys into the call's (agent-scope atomics on the
// keys of the argmax state); the last workgroup of the launch (a ticket
// counter) decodes the keys of its tokens into index and value and clears
// keys and counter for the next call.  tok0: the launch's first token.
template <int MT>
__device__ void argmax_finish(unsigned long long *key, uint32_t *count, int32_t *index, float *value, int tok0,
                              const unsigned long long *best)
{
#pragma unroll
    for (int m = 0; m < MT; m++)
        __hip_atomic_fetch_max(&key[tok0 + m], best[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t total = gridDim.x * gridDim.y;
    const uint32_t ticket = __hip_atomic_fetch_add(count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket != total - 1)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const unsigned long long k = __hip_atomic_load(&key[tok0 + m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t ord = (uint32_t)(k >> 32);
        const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
        index[tok0 + m] = (int32_t)(~(uint32_t)k);
        value[tok0 + m] = __uint_as_float(u);
        __hip_atomic_store(&key[tok0 + m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Passes in flight per wavefront besides the one computed.  Two is the
// measured optimum on MI355X (same-box runs of the 9B and 1B decode steps):
// three cost 3.5% and four 10% more per step, one 3% more; more requests in
// flight per compute unit raise every load's latency more than they hide.
constexpr int kDepth = 2;

template <int MT, int OM, int KP, int RS>
__device__ __forceinline__ void plan_body(const u32x16 a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t *plan = (const uint8_t *)u64_ptr(a[0], a[1]);
    void *const yptr = (void *)u64_ptr(a[2], a[3]);
    const uint16_t *xptr = (const uint16_t *)u64_ptr(a[4], a[5]);
    const uint32_t region_bytes = a[6];
    const int Nm = (int)a[7], ldy = (int)a[8], rows = (int)a[9], ldx = (int)a[10];
    const int passes = (int)a[11], per_wave = (int)a[12];
    const int G = (int)(a[13] & 0xffffu), yt = (int)(a[13] >> 16);
    const int smax = (int)a[15];
    const int blk = (int)blockIdx.x;
    const int n0 = blk * rows;
    const int R = min(rows, Nm - n0);
    const int stride = pos_stride(rows, G);
    const PLayout L = p_layout(MT, G, smax);
    const int ps = psum_stride(G, smax);
    uint32_t *xrec = reinterpret_cast<uint32_t *>(smem + L.x);
    float *psum = reinterpret_cast<float *>(smem + L.psum);
    float *ybuf = reinterpret_cast<float *>(smem + L.ybuf);
    unsigned long long *best = reinterpret_cast<unsigned long long *>(smem + L.best);
    const YOut yo{yptr, ldy, n0, yt, smax, best};
    // the block's region as a buffer resource: pass p's loads are an SGPR
    // offset (1536 p) away from the same per-lane offsets
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(plan + (uint64_t)blk * region_bytes), 0, (int)region_bytes, 0x00020000);
    const int voff_c = lane * 16, voff_w = kCodeArea + lane * 8;
    // Loads past this wavefront's last pass (the pipeline runs kDepth + 1
    // passes ahead; before the width bytes are in, past the plan's pass count)
    // go through an empty resource: they are issued, so every wait stays
    // exact, and return zeros without a memory access.
    const __amdgpu_buffer_rsrc_t r0 = __builtin_amdgcn_make_buffer_rsrc((void *)plan, 0, 0, 0x00020000);
    // width bytes of this wavefront's passes (lane i < per_wave / 4: passes
    // 4i..4i+3 of the wave; the other lanes hold zeros)
    const bool own = lane < (per_wave >> 2);
    const uint32_t meta_raw =
        __builtin_amdgcn_raw_buffer_load_b32(rs, own ? lane * 4 : 0, passes * kPassBytes + wave * per_wave, 0);
    const uint32_t meta = own ? meta_raw : 0u;
    // activations: their loads go out first, so that waiting for them leaves
    // the pass loads below in flight
    XRegs<KP> xs;
    x_load<MT, KP>(xptr, ldx, G, xs);
    int npw = (passes - wave + kW - 1) / kW; // this wavefront's pass count (an upper bound until its width bytes are in)
    auto issue = [&](PBuf &b, int i) {
        const bool own = i < npw;
        const __amdgpu_buffer_rsrc_t r = own ? rs : r0;
        const int p = own ? wave + kW * i : 0;
        b.c = __builtin_amdgcn_raw_buffer_load_b128(r, voff_c, p * kPassBytes, 0);
        b.w = __builtin_amdgcn_raw_buffer_load_b64(r, voff_w, p * kPassBytes, 0);
    };
    // in the order the loop issues them (codes, then words, pass by pass), so
    // that its waits are the same on the first trip as on every later one.
    // The first two passes go out before the activations are staged, the
    // third after the barrier: with more pass loads of every wavefront of the
    // device in flight, the activation loads queue behind them and the first
    // barrier comes late (measured: two ahead is 7% faster on a 9B step, 10%
    // on a 1B step, than four ahead, and also faster than none; one ahead
    // and two after is the same as two and one)
    PBuf b0, b1, b2;
    issue(b0, 0);
    asm volatile("" ::: "memory");
    issue(b1, 1);
    asm volatile("" ::: "memory");
    x_store<MT, KP>(G, xs, xrec);
    if (tid < MT)
        best[tid] = 0ull;
    __syncthreads();
    issue(b2, 2);

    const PCtx cx{xrec, psum, G, ps, 0xffffffffu / (uint32_t)stride + 1u};
    // passes of this wavefront: its width bytes are nonzero up to the first 0
    // (lane i holds bytes 4i..4i+3, and the list ends inside its own lanes),
    // so full lanes form a prefix
    const int cl = (meta & 0xffu) ? ((meta & 0xff00u) ? ((meta & 0xff0000u) ? ((meta >> 24) ? 4 : 3) : 2) : 1) : 0;
    const int nfull = __popcll(__ballot(cl == 4));
    npw = 4 * nfull + __builtin_amdgcn_readlane(cl, nfull);
    // pass i: the pass body, then (always, so that every step issues the same
    // loads and the waits stay exact) the loads of pass i + 4 into the same
    // registers
    auto step = [&](PBuf &b, int i) {
        if (i < npw) {
            const uint32_t mw = (uint32_t)__builtin_amdgcn_readlane((int)meta, i >> 2);
            switch ((mw >> (8 * (i & 3))) & 0xffu) {
            case 1: pass_b1<MT>(b, cx); break;
            case 2: pass_b2<MT>(b, cx); break;
            case 3: pass_b4<MT>(b, cx); break;
            default: pass_b8<MT>(b, cx); break;
            }
        }
        issue(b, i + kDepth + 1);
    };
    for (int i = 0; i < npw; i += 3) {
        step(b0, i);
        step(b1, i + 1);
        step(b2, i + 2);
    }
    __syncthreads(); // every partial of the block is in psum

    row_sums<MT, OM, RS>(wave, R, stride, G, ps, psum, ybuf, yo);
    if constexpr (OM == kArgmax) {
        __syncthreads(); // every row's key is in best[]
        if (tid == 0) {
            // argmax launches: y is the state (16 keys, then the counter);
            // the second record holds the index and value outputs
            const u32x16 o = kernarg_line((uint32_t)sizeof(PRec));
            unsigned long long *key = reinterpret_cast<unsigned long long *>(yptr);
            argmax_finish<MT>(key, reinterpret_cast<uint32_t *>(key + 16), (int32_t *)u64_ptr(o[0], o[1]),
                              (float *)u64_ptr(o[2], o[3]), ldy, best);
        }
    } else if constexpr (OM == kSwiglu) {
        __syncthreads(); // every row of the block is in ybuf
        const int pairs = R / 2; // R is even: the block starts at an even row and N is even
        for (int i = tid; i < MT * pairs; i += kT) {
            const int m = i / pairs, p = i - m * pairs;
            const float g = ybuf[m * smax + 2 * p], u = ybuf[m * smax + 2 * p + 1];
            const float h = g / (1.0f + expf(-g)) * u; // silu(gate) * up
            const uint64_t o = (uint64_t)m * ldy + n0 / 2 + p;
            if (yt == VBQ_F16)
                ((gu16_t *)yptr)[o] = __half_as_ushort(__float2half_rn(h));
            else
                ((gf32_t *)yptr)[o] = h;
        }
    }
}

template <int MT, int OM, int KP>
__global__ __launch_bounds__(kT) void k_gemv_plan(PArgs /* read through kernarg_line */)
{
    // this workgroup's record (matrix blockIdx.y of the launch), in one load
    const u32x16 a = kernarg_line((uint32_t)blockIdx.y * (uint32_t)sizeof(PRec));
    if ((int)blockIdx.x >= (int)a[14])
        return; // the launch spans the largest matrix; a smaller one has fewer blocks
    plan_body<MT, OM, KP, 0>(a);
}

// One matrix, one token, plain rows or the SwiGLU epilogue: the record's fields
// as scalar arguments, which the dispatch preloads into SGPRs, so no wavefront
// waits for a load of its arguments.  RS: the row shape (row_shape_of(G)).
template <int OM, int KP, int RS>
__global__ __launch_bounds__(kT) void k_gemv_plan1(const uint8_t *plan, void *y, const uint16_t *x, uint32_t region,
                                                   int N, int rows, int passes, int per_wave, uint32_t g_yt, int smax)
{
    u32x16 a;
    a[0] = (uint32_t)(uintptr_t)plan;
    a[1] = (uint32_t)((uintptr_t)plan >> 32);
    a[2] = (uint32_t)(uintptr_t)y;
    a[3] = (uint32_t)((uintptr_t)y >> 32);
    a[4] = (uint32_t)(uintptr_t)x;
    a[5] = (uint32_t)((uintptr_t)x >> 32);
    a[6] = region;
    a[7] = (uint32_t)N;
    a[8] = 0u; // ldy: one token
    a[9] = (uint32_t)rows;
    a[10] = 0u; // ldx: one token
    a[11] = (uint32_t)passes;
    a[12] = (uint32_t)per_wave;
    a[13] = g_yt;
    a[14] = 0x7fffffffu;
    a[15] = (uint32_t)smax;
    plan_body<1, OM, KP, RS>(a);
}

// Two matrices of one shape that share x (a layer's gate and up projections),
// one token, plain rows: both records in 13 preloaded scalar arguments
// (n_rows = N | rows << 20, passes = passes of matrix 0 | of matrix 1 << 16;
// per-wave bytes, region and position stride follow from them); blockIdx.y
// picks the matrix.
template <int KP, int RS>
__global__ __launch_bounds__(kT) void k_gemv_plan2(const uint8_t *plan0, const uint8_t *plan1, void *y0, void *y1,
                                                   const uint16_t *x, uint32_t n_rows, uint32_t passes01, uint32_t g_yt)
{
    const bool second = blockIdx.y != 0;
    const uint8_t *plan = second ? plan1 : plan0;
    void *y = second ? y1 : y0;
    const int passes = (int)(second ? passes01 >> 16 : passes01 & 0xffffu);
    const int per_wave = per_wave_for(passes), rows = (int)(n_rows >> 20);
    u32x16 a;
    a[0] = (uint32_t)(uintptr_t)plan;
    a[1] = (uint32_t)((uintptr_t)plan >> 32);
    a[2] = (uint32_t)(uintptr_t)y;
    a[3] = (uint32_t)((uintptr_t)y >> 32);
    a[4] = (uint32_t)(uintptr_t)x;
    a[5] = (uint32_t)((uintptr_t)x >> 32);
    a[6] = region_for(passes, per_wave);
    a[7] = n_rows & 0xfffffu;
    a[8] = 0u; // ldy: one token
    a[9] = (uint32_t)rows;
    a[10] = 0u; // ldx: one token
    a[11] = (uint32_t)passes;
    a[12] = (uint32_t)per_wave;
    a[13] = g_yt;
    a[14] = 0x7fffffffu; // both matrices have the launch's block count
    a[15] = (uint32_t)pos_stride(rows, (int)(g_yt & 0xffffu));
    plan_body<1, kRows, KP, RS>(a);
}

// ---------------------------------------------------------------------------
// Host side.

uint64_t region_of(int passes, int per_wave) { return region_for(passes, per_wave); }

int per_wave_of(int passes) { return per_wave_for(passes); }

vbq_status check_plan(const vbq_plan *P)
{
    if (!P || P->magic != VBQ_PLAN_MAGIC)
        return VBQ_ERR_LAYOUT;
    if (P->N < 1 || P->G < 1 || P->G > kMaxG || P->K != 64 * P->G || P->M < 1 || P->M > 2 || P->wgs < 1 ||
        P->rows < 1 || (int64_t)P->wgs * P->rows < P->N || (int64_t)(P->wgs - 1) * P->rows >= P->N ||
        P->wgs > 65535 || P->passes < 1 || P->per_wave != per_wave_of(P->passes) || P->per_wave > kMaxPerWave ||
        (int64_t)pos_stride(P->rows, P->G) * P->G + 1 > 65536 ||
        P->psum != psum_stride(P->G, pos_stride(P->rows, P->G)) ||
        P->region_bytes != region_of(P->passes, P->per_wave) ||
        P->total_bytes != (uint64_t)P->wgs * P->region_bytes)
        return VBQ_ERR_LAYOUT;
    return VBQ_OK;
}

PrepArgs prep_args(const vbq_layout *L, const void *blob, const vbq_plan *P)
{
    PrepArgs a{};
    a.blob = (const uint8_t *)blob;
    a.off_row_off = L->off_row_off;
    a.off_slice_off = L->off_slice_off;
    a.off_wmap = L->off_wmap;
    a.off_scales = L->off_scales;
    a.off_codes = L->off_codes;
    a.N = (int)L->N;
    a.G = (int)L->G;
    a.nS = (int)L->nS;
    a.rows = P->rows;
    a.passes = P->passes;
    a.per_wave = P->per_wave;
    a.region = P->region_bytes;
    return a;
}

vbq_status lds_attribute_once(const void *fn) { return dynamic_lds_once(fn, kLdsBudget); }

// f(std::integral_constant<int, RS>) for the row shape rs of a one-token
// launch whose activation staging takes KP items per thread (KP = 1: G <= 256,
// L = 8, 16 or 32; KP = 2: L = 64); false if rs is not one of them.
template <int KP, typename F>
bool with_row_shape(int rs, F &&f, vbq_status &st)
{
#define VBQ_RS(S_)                                                                                                  \
    case S_: st = f(std::integral_constant<int, S_>{}); return true;
    if constexpr (KP == 1) {
        switch (rs) {
            VBQ_RS(8 * 16 + 8) VBQ_RS(8 * 16 + 7) VBQ_RS(8 * 16 + 4) VBQ_RS(8 * 16)
            VBQ_RS(16 * 16 + 8) VBQ_RS(16 * 16 + 7) VBQ_RS(16 * 16)
            VBQ_RS(32 * 16 + 8) VBQ_RS(32 * 16 + 7) VBQ_RS(32 * 16)
        }
    } else if constexpr (KP == 2) {
        switch (rs) { VBQ_RS(64 * 16 + 8) VBQ_RS(64 * 16 + 7) VBQ_RS(64 * 16) }
    }
#undef VBQ_RS
    return false;
}

template <int MT, int OM, int KP>
vbq_status launch_plan_t(const PArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    vbq_status st = VBQ_OK;
    if constexpr (MT == 1 && (OM == kRows || OM == kSwiglu)) {
        if (grid.y == 1) {
            const PRec &r = a.rec[0];
            auto go = [&](auto rsc) -> vbq_status {
                constexpr int RS = decltype(rsc)::value;
                VBQ_TRY(lds_attribute_once((const void *)k_gemv_plan1<OM, KP, RS>));
                hipLaunchKernelGGL((k_gemv_plan1<OM, KP, RS>), dim3(grid), dim3(kT), lds, stream, r.plan, r.y, r.x,
                                   r.region, r.N, r.rows, r.passes, r.per_wave, r.g_yt, r.smax);
                return launch_status();
            };
            if (with_row_shape<KP>(row_shape_of((int)(r.g_yt & 0xffffu)), go, st))
                return st;
        }
    }
    if constexpr (MT == 1 && OM == kRows) {
        const PRec &r0 = a.rec[0], &r1 = a.rec[1];
        const int G = (int)(r0.g_yt & 0xffffu);
        if (grid.y == 2 && r0.x == r1.x && r0.g_yt == r1.g_yt && r0.N == r1.N && r0.rows == r1.rows &&
            r0.wgs == (int)grid.x && r1.wgs == (int)grid.x && r0.N < (1 << 20) && r0.rows < (1 << 12) &&
            r0.passes < (1 << 16) && r1.passes < (1 << 16) && r0.smax == pos_stride(r0.rows, G) &&
            r0.smax == r1.smax) {
            auto go = [&](auto rsc) -> vbq_status {
                constexpr int RS = decltype(rsc)::value;
                VBQ_TRY(lds_attribute_once((const void *)k_gemv_plan2<KP, RS>));
                hipLaunchKernelGGL((k_gemv_plan2<KP, RS>), dim3(grid), dim3(kT), lds, stream, r0.plan, r1.plan, r0.y,
                                   r1.y, r0.x, (uint32_t)r0.N | ((uint32_t)r0.rows << 20),
                                   (uint32_t)r0.passes | ((uint32_t)r1.passes << 16), r0.g_yt);
                return launch_status();
            };
            if (with_row_shape<KP>(row_shape_of(G), go, st))
                return st;
        }
    }
    VBQ_TRY(lds_attribute_once((const void *)k_gemv_plan<MT, OM, KP>));
    hipLaunchKernelGGL((k_gemv_plan<MT, OM, KP>), dim3(grid), dim3(kT), lds, stream, a);
    return launch_status();
}

template <int MT, int OM>
vbq_status launch_plan_kp(int G, const PArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    const int per = (MT * G * 4 + kT - 1) / kT; // activation items per thread
    if (per <= 1)
        return launch_plan_t<MT, OM, 1>(a, grid, lds, stream);
    if (per <= 2)
        return launch_plan_t<MT, OM, 2>(a, grid, lds, stream);
    if (per <= 4)
        return launch_plan_t<MT, OM, 4>(a, grid, lds, stream);
    return launch_plan_t<MT, OM, 8>(a, grid, lds, stream);
}

// One launch of m (1 or 2) tokens in output mode om.
vbq_status launch_plan(int m, int om, const PArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    const int G = (int)(a.rec[0].g_yt & 0xffffu);
    switch (om * 2 + (m - 1)) {
    case 0: return launch_plan_kp<1, kRows>(G, a, grid, lds, stream);
    case 1: return launch_plan_kp<2, kRows>(G, a, grid, lds, stream);
    case 2: return launch_plan_kp<1, kArgmax>(G, a, grid, lds, stream);
    case 3: return launch_plan_kp<2, kArgmax>(G, a, grid, lds, stream);
    case 4: return launch_plan_kp<1, kSwiglu>(G, a, grid, lds, stream);
    default: return launch_plan_kp<2, kSwiglu>(G, a, grid, lds, stream);
    }
}

bool lds_fits(int M, int G, int rows)
{
    return p_layout(M, G, pos_stride(rows, G)).total <= kLdsBudget && (int64_t)pos_stride(rows, G) * G + 1 <= 65536;
}

} // namespace

bool vbq::planned_can_share(const vbq_plan *a, const vbq_plan *b)
{
    return a->K == b->K && a->M == b->M &&
           lds_fits(a->M, a->G, std::max(pos_stride(a->rows, a->G), pos_stride(b->rows, b->G)));
}

extern "C" {

vbq_status vbq_plan_init(const vbq_layout *L, const void *blob, int M, int wgs, vbq_plan *P, void *ws,
                         size_t ws_bytes, hipStream_t stream)
{
    if (!blob || !P)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    if (M < 1 || M > 2)
        return VBQ_ERR_BATCH;
    if (!ws || ws_bytes < 16)
        return VBQ_ERR_WORKSPACE;
    if ((uintptr_t)blob % 256 || (uintptr_t)ws % 4)
        return VBQ_ERR_ALIGN;
    const int N = (int)L->N, G = (int)L->G;
    if (G > kMaxG)
        return VBQ_ERR_SHAPE;
    const int cus = current_device_cus();
    if (wgs <= 0)
        wgs = cus;
    // rows per block: an even count whenever N is even, so that a row block
    // never splits the (gate, up) pairs of an interleaved SwiGLU matrix; fewer
    // rows (more blocks) while a block's partial sums do not fit the LDS
    auto fit = [&](int m, int &rows_out) {
        const int step = N % 2 == 0 ? 2 : 1; // an even N keeps even blocks
        int rows = (N + wgs - 1) / wgs;
        rows += rows % step;
        for (;;) {
            if (lds_fits(m, G, rows)) {
                rows_out = rows;
                return true;
            }
            if (rows <= step)
                return false;
            // about 3/4 as many rows, a multiple of step, and strictly fewer
            rows = std::max(step, std::min(rows - step, rows * 3 / 4 / step * step));
        }
    };
    int rows = 0;
    if (M == 2 && !(fit(2, rows) && (N + rows - 1) / rows <= 4 * cus))
        M = 1; // two tokens would need many rounds of small blocks: one token per launch
    if (M == 1 && !fit(1, rows))
        return VBQ_ERR_SHAPE;
    wgs = (N + rows - 1) / rows;
    if (wgs > 65535)
        return VBQ_ERR_SHAPE;
    vbq_plan p{};
    p.magic = VBQ_PLAN_MAGIC;
    p.N = N;
    p.K = (int)L->K;
    p.G = G;
    p.M = M;
    p.wgs = wgs;
    p.rows = rows;
    p.psum = psum_stride(G, pos_stride(rows, G));
    p.lds_bytes = (int)p_layout(M, G, pos_stride(rows, G)).total;
    // sizing pass: the largest block's pass count
    VBQ_TRY(zero_words(ws, 16, stream));
    PrepArgs a = prep_args(L, blob, &p);
    a.plan = nullptr;
    a.sizes = (uint32_t *)ws;
    hipLaunchKernelGGL(k_prepare, dim3(wgs), dim3(kT), 0, stream, a);
    VBQ_TRY(launch_status());
    uint32_t h[4];
    VBQ_TRY(hip_status(hipMemcpyAsync(h, ws, 16, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipStreamSynchronize(stream)));
    if (h[0] < 1 || h[0] > (uint32_t)kW * (kMaxPerWave - 4))
        return VBQ_ERR_SHAPE;
    p.passes = (int)h[0];
    p.per_wave = per_wave_of(p.passes);
    p.region_bytes = region_of(p.passes, p.per_wave);
    p.total_bytes = (uint64_t)wgs * p.region_bytes;
    *P = p;
    return VBQ_OK;
}

vbq_status vbq_prepare(const vbq_plan *P, const vbq_layout *L, const void *blob, void *plan, uint32_t *status_word,
                       hipStream_t stream)
{
    if (!blob || !plan)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    VBQ_TRY(check_plan(P));
    if ((int)L->N != P->N || (int)L->K != P->K)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)blob % 256 || (uintptr_t)plan % 256 || (uintptr_t)status_word % 4)
        return VBQ_ERR_ALIGN;
    if (status_word)
        VBQ_TRY(zero_words(status_word, 4, stream));
    PrepArgs a = prep_args(L, blob, P);
    a.plan = (uint8_t *)plan;
    a.sizes = nullptr;
    a.status = status_word;
    hipLaunchKernelGGL(k_prepare, dim3(P->wgs), dim3(kT), 0, stream, a);
    return launch_status();
}

} // extern "C"

namespace {

// Checks one launch for up to P->M tokens and fills its arguments; launches nothing.
vbq_status planned_args(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                        int tok0, PArgs *out, dim3 *grid_out, uint32_t *lds_out)
{
    if ((uintptr_t)x % 8 || ldx % 4)
        return VBQ_ERR_ALIGN; // the activations are read 8 bytes at a time
    if ((int64_t)(M - 1) * ldx + items[0].P->K >= (int64_t)1 << 30)
        return VBQ_ERR_SHAPE; // one launch's activations are addressed with 32-bit byte offsets
    PArgs a{};
    int gx = 0, smax = 2;
    for (int i = 0; i < n; i++) {
        const vbq_planned_item &it = items[i];
        if (!it.P || !it.plan || !it.y)
            return VBQ_ERR_INVALID_ARG;
        VBQ_TRY(check_plan(it.P));
        const vbq_plan *P = it.P;
        const vbq_plan *P0 = items[0].P;
        if (M > P->M)
            return VBQ_ERR_BATCH;
        if (P->K != P0->K || ldx < P->K || it.ldy < P->N)
            return VBQ_ERR_SHAPE;
        if ((uintptr_t)it.plan % 256 || (uintptr_t)it.y % (yt == VBQ_F32 ? 4 : 2))
            return VBQ_ERR_ALIGN;
        PRec &r = a.rec[i];
        r.plan = (const uint8_t *)it.plan;
        r.y = (uint8_t *)it.y + (uint64_t)tok0 * it.ldy * (yt == VBQ_F32 ? 4 : 2);
        r.x = x + (uint64_t)tok0 * ldx;
        r.region = (uint32_t)P->region_bytes;
        r.N = P->N;
        r.ldy = it.ldy;
        r.rows = P->rows;
        r.ldx = ldx;
        r.passes = P->passes;
        r.per_wave = P->per_wave;
        r.wgs = P->wgs;
        gx = std::max(gx, P->wgs);
        smax = std::max(smax, pos_stride(P->rows, P->G)); // LDS strides: the plan with the most rows fits
    }
    const int G = items[0].P->G;
    const uint32_t lds = p_layout(M, G, smax).total;
    if (lds > kLdsBudget || (int64_t)smax * G + 1 > 65536)
        return VBQ_ERR_SHAPE;
    for (int i = 0; i < n; i++) {
        PRec &r = a.rec[i];
        r.g_yt = (uint32_t)G | (uint32_t)yt << 16;
        r.smax = smax;
    }
    *out = a;
    *grid_out = dim3((unsigned)gx, (unsigned)n);
    *lds_out = lds;
    return VBQ_OK;
}

// Tokens beyond what one launch holds run as further launches over the same
// plans; each token's arithmetic is the same in every launch shape.  Every
// launch is checked before the first is enqueued; with dry set, only the
// checks run.
vbq_status planned_shared(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                          hipStream_t stream, bool dry)
{
    if (!items || n < 1 || n > VBQ_MAX_SHARED || !x)
        return VBQ_ERR_INVALID_ARG;
    if (yt != VBQ_F32 && yt != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    int chunk = 2;
    for (int i = 0; i < n; i++) {
        if (!items[i].P)
            return VBQ_ERR_INVALID_ARG;
        VBQ_TRY(check_plan(items[i].P));
        chunk = std::min(chunk, (int)items[i].P->M);
    }
    PArgs a;
    dim3 grid;
    uint32_t lds;
    for (int pass = 0; pass < (dry ? 1 : 2); pass++)
        for (int t0 = 0; t0 < M; t0 += chunk) {
            const int m = std::min(chunk, M - t0);
            VBQ_TRY(planned_args(items, n, m, x, ldx, yt, t0, &a, &grid, &lds));
            if (pass == 1)
                VBQ_TRY(launch_plan(m, kRows, a, grid, lds, stream));
        }
    return VBQ_OK;
}

} // namespace

vbq_status vbq::planned_shared_check(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                     vbq_dtype yt)
{
    return planned_shared(items, n, M, x, ldx, yt, nullptr, true);
}

extern "C" {

vbq_status vbq_gemv_planned_shared(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                   vbq_dtype yt, hipStream_t stream)
{
    return planned_shared(items, n, M, x, ldx, yt, stream, false);
}

vbq_status vbq_gemv_planned(const vbq_plan *P, const void *plan, int M, const uint16_t *x, int ldx, void *y, int ldy,
                            vbq_dtype yt, hipStream_t stream)
{
    const vbq_planned_item it{P, plan, y, ldy};
    return vbq_gemv_planned_shared(&it, 1, M, x, ldx, yt, stream);
}

vbq_status vbq_gemv_planned_swiglu(const vbq_plan *P, const void *plan, int M, const uint16_t *x, int ldx, void *h,
                                   int ldh, vbq_dtype ht, hipStream_t stream)
{
    if (!P || !plan || !x || !h)
        return VBQ_ERR_INVALID_ARG;
    if (ht != VBQ_F32 && ht != VBQ_F16)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    VBQ_TRY(check_plan(P));
    if (P->N % 2 || P->rows % 2 || ldh < P->N / 2)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)h % (ht == VBQ_F32 ? 4 : 2))
        return VBQ_ERR_ALIGN;
    const int chunk = P->M;
    const int esz = ht == VBQ_F32 ? 4 : 2;
    // an ordinary planned GEMV's checks and arguments (outputs of width N / 2
    // would fail its ldy >= N check, so it sees ldy = N), then the output
    // switched to the pairs
    const vbq_planned_item it{P, plan, h, P->N};
    PArgs a;
    dim3 grid;
    uint32_t lds;
    for (int pass = 0; pass < 2; pass++)
        for (int t0 = 0; t0 < M; t0 += chunk) {
            const int m = std::min(chunk, M - t0);
            VBQ_TRY(planned_args(&it, 1, m, x, ldx, ht, t0, &a, &grid, &lds));
            a.rec[0].y = (uint8_t *)h + (uint64_t)t0 * (uint64_t)ldh * (uint64_t)esz;
            a.rec[0].ldy = ldh;
            if (pass == 1)
                VBQ_TRY(launch_plan(m, kSwiglu, a, grid, lds, stream));
        }
    return VBQ_OK;
}

} // extern "C"

vbq_status vbq::planned_argmax(const vbq_plan *P, const void *plan, int M, const uint16_t *x, int ldx, void *state,
                               int32_t *index, float *value, hipStream_t stream)
{
    const int chunk = P->M;
    // the same checks and arguments as an fp32 planned GEMV writing to the
    // state, then the record is switched to the argmax output (y = state,
    // ldy = first token, outputs in the second record)
    const vbq_planned_item it{P, plan, state, P->N};
    PArgs a;
    dim3 grid;
    uint32_t lds;
    for (int pass = 0; pass < 2; pass++)
        for (int t0 = 0; t0 < M; t0 += chunk) {
            const int m = std::min(chunk, M - t0);
            VBQ_TRY(planned_args(&it, 1, m, x, ldx, VBQ_F32, t0, &a, &grid, &lds));
            a.rec[0].y = state;
            a.rec[0].ldy = t0;
            a.rec[1].plan = (const uint8_t *)index;
            a.rec[1].y = value;
            if (pass == 1)
                VBQ_TRY(launch_plan(m, kArgmax, a, grid, lds, stream));
        }
    return VBQ_OK;
}

extern "C" {

vbq_status vbq_gemv_planned_argmax(const vbq_plan *P, const void *plan, int M, const uint16_t *x, int ldx,
                                   vbq_argmax_ws *ws, hipStream_t stream)
{
    if (!P || !plan || !x || !ws)
        return VBQ_ERR_INVALID_ARG;
    if (M < 1 || M > 16)
        return VBQ_ERR_BATCH;
    VBQ_TRY(check_plan(P));
    if ((uintptr_t)ws % 8)
        return VBQ_ERR_ALIGN;
    return planned_argmax(P, plan, M, x, ldx, ws, ws->index, ws->value, stream);
}

} // extern "C"
