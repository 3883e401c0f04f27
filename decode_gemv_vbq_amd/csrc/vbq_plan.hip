// Prepared GEMV plans: a one-time device re-encoding of a VBQ1 matrix into
// the order in which the decode kernel consumes it, and that kernel.
//
// The method ("Variable Bit-width Quantization", mlsanity.com page, Abstract)
// gives every contiguous group of 64 weights its own width in {1,2,4,8}, and
// decode multiplies the packed codes without materialising the weights.  The
// VBQ1 blob stores groups row by row, bucketed by width inside each 32-group
// slice.  A wavefront must run 64 groups of ONE width at a time, so a kernel
// reading VBQ1 directly has to plan each tile at run time (find every group
// of each width, assign it a slot) before it can compute.  A plan moves that
// work to a preparation step that runs once per matrix:
//
//  * The rows are split into row blocks, one per workgroup of the GEMV launch.
//    Each block owns a fixed-size region of the plan buffer holding tiles at
//    a fixed stride.  Tile t takes the groups (row-major order over the
//    block) whose running byte count starts in [t*C, (t+1)*C), so a row may
//    continue in the next tile.
//  * Inside a tile, groups are sorted by (width 8,4,2,1; group column; row).
//    The tile stores a 64-byte header, the code records in that order
//    (verbatim 8*b bytes each, so each width section starts aligned to its
//    record size), and one 32-bit word per group: its fp16 scale and the
//    group's position e = column * rows_in_tile + row_in_tile.
//  * Each header carries the byte size of the next tile, and the plan carries
//    the largest first tile, so the kernel issues every copy without first
//    reading metadata.
//
// The GEMV kernel: one 1024-thread workgroup per row block.  As soon as the
// kernel starts, half of the workgroup copies tile 0 into LDS with
// global_load_lds_dwordx4 while the other half stages the activations.  Tile
// k+1 is copied by two waves into the other half of a two-slot ring while the
// other waves run the passes of tile k, handed out through an LDS counter;
// then every wave sums the rows of tile k-1.  One barrier per tile.  A pass is
// 64 slots of one width: codes are contiguous per lane, x is read per group
// column (lanes of a column broadcast), partials land at e (contiguous per
// column).  Row sums follow the column order and the tile order, so the
// result does not depend on timing.
#include <algorithm>

#include "vbq_common.h"
#include "vbq_host.h"
#include "vbq_unpack.h"

using namespace vbq;

namespace {

constexpr int kT = 1024; // threads per workgroup (prepare and GEMV kernels)
constexpr int kW = kT / 64;
constexpr int kHdr = 64;    // tile header bytes
constexpr int kXRec = 36;   // dwords of x per group: 32 pairs (x_p, x_{p+32}) + 4 constants
constexpr int kMaxG = 512;  // groups per row the plans support (K <= 32768)
constexpr int kMaxTiles = 1024; // tiles per row block
constexpr int kMaxMats = VBQ_MAX_SHARED;
constexpr int kMaxTb = 64 * 1024; // tile stride bound (16-bit positions)
constexpr int kCopyWaves = 2;     // waves of the GEMV workgroup that copy the next tile

// Usable bytes per tile before the last group's overhang: a group starting
// below C ends at most 68 bytes later, and the header takes 64.
__host__ __device__ constexpr uint32_t tile_cut(uint32_t tb) { return tb - kHdr - 68u; }

// Bytes a group of width code c occupies in a tile: code record + scale/position word.
__device__ __forceinline__ uint32_t group_bytes(int c) { return (8u << c) + 4u; }

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
    uint32_t tb;     // tile stride
    uint64_t region; // bytes per block region
    uint8_t *plan;   // null: sizing only
    uint32_t *sizes; // sizing: [0] max tiles, [1] max first-tile bytes, [2] blocks over kMaxTiles
};

// LDS of the preparation kernel.
struct PrepShared {
    uint32_t tmp[kW + 1];
    uint32_t sizes[kT];                // group sizes of the current chunk
    uint32_t carry, prev_size, ntiles;
    uint32_t tstart[kMaxTiles + 1];    // first group of each tile
    uint32_t tcum[kMaxTiles + 1];      // running byte count at each tile start
    uint32_t hist[4 * kMaxG];          // per (section, column): count, then first slot
};

// One workgroup per row block: tile boundaries from a running byte count over
// the block's groups in row-major order; then (plan != null) each tile is
// written: groups counted per (width, column), given slots in (width 8,4,2,1;
// column; row) order, and their code records, scales and positions copied.
__global__ __launch_bounds__(kT) void k_prepare(PrepArgs a)
{
    __shared__ PrepShared sh;
    const int tid = threadIdx.x;
    const int n0 = (int)blockIdx.x * a.rows;
    if (n0 >= a.N)
        return;
    const int R = min(a.rows, a.N - n0);
    const int G = a.G;
    const uint32_t NG = (uint32_t)R * (uint32_t)G;
    const uint32_t C = tile_cut(a.tb);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap);
    if (tid == 0) {
        sh.carry = 0;
        sh.prev_size = 0;
        sh.ntiles = 0;
    }
    __syncthreads();
    // ---- tile boundaries: group i starts tile t = floor(start_i / C) when the
    // previous group started in an earlier tile
    for (uint32_t base = 0; base < NG; base += kT) {
        const uint32_t i = base + (uint32_t)tid;
        uint32_t s = 0;
        if (i < NG) {
            const int r = (int)(i / (uint32_t)G), g = (int)(i - (uint32_t)r * G);
            s = group_bytes(vbq1_width(wmap, a.nS, n0 + r, g));
        }
        sh.sizes[tid] = s;
        const uint32_t carry = sh.carry, prev_size = sh.prev_size;
        uint32_t total;
        const uint32_t ex = block_excl_scan(s, sh.tmp, total); // (its barriers publish sizes[])
        if (i < NG) {
            const uint32_t start = carry + ex;
            const uint32_t t = start / C;
            const uint32_t sp = tid ? sh.sizes[tid - 1] : prev_size; // size of group i-1
            if (i == 0 || (start - sp) / C < t) {
                if (t < (uint32_t)kMaxTiles) {
                    sh.tstart[t] = i;
                    sh.tcum[t] = start;
                }
                atomicMax(&sh.ntiles, t + 1);
            }
        }
        __syncthreads();
        if (tid == 0) {
            sh.carry = carry + total;
            const uint32_t last = min(NG - base, (uint32_t)kT) - 1;
            sh.prev_size = sh.sizes[last];
        }
        __syncthreads();
    }
    const uint32_t total_bytes = sh.carry;
    const uint32_t ntiles = sh.ntiles;
    if (ntiles > (uint32_t)kMaxTiles) {
        if (tid == 0 && a.sizes)
            atomicAdd(a.sizes + 2, 1u);
        return;
    }
    if (tid == 0) {
        sh.tstart[ntiles] = NG;
        sh.tcum[ntiles] = total_bytes;
    }
    __syncthreads();
    if (!a.plan) {
        if (tid == 0) {
            atomicMax(a.sizes, ntiles);
            atomicMax(a.sizes + 1, (uint32_t)kHdr + sh.tcum[1] - sh.tcum[0]);
        }
        return;
    }
    // ---- tiles
    const uint32_t *rowoff = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off);
    const uint32_t *sloff = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off);
    const uint16_t *scales = reinterpret_cast<const uint16_t *>(a.blob + a.off_scales);
    const uint8_t *codes = a.blob + a.off_codes;
    uint8_t *region = a.plan + (uint64_t)blockIdx.x * a.region;
    for (uint32_t t = 0; t < ntiles; t++) {
        const uint32_t i0 = sh.tstart[t], i1 = sh.tstart[t + 1];
        const int ra = (int)(i0 / (uint32_t)G), rb = (int)((i1 - 1) / (uint32_t)G);
        const int NR = rb - ra + 1;
        for (int k = tid; k < 4 * G; k += kT)
            sh.hist[k] = 0;
        __syncthreads();
        for (uint32_t i = i0 + (uint32_t)tid; i < i1; i += kT) {
            const int r = (int)(i / (uint32_t)G), g = (int)(i - (uint32_t)r * G);
            const int c = vbq1_width(wmap, a.nS, n0 + r, g);
            atomicAdd(&sh.hist[(3 - c) * G + g], 1u); // sections 8,4,2,1
        }
        __syncthreads();
        // exclusive prefix over (section, column): first slot of each bucket
        {
            uint32_t carry = 0;
            for (int base = 0; base < 4 * G; base += kT) {
                const int k = base + tid;
                const uint32_t v = k < 4 * G ? sh.hist[k] : 0u;
                uint32_t tot;
                const uint32_t ex = block_excl_scan(v, sh.tmp, tot);
                if (k < 4 * G)
                    sh.hist[k] = carry + ex;
                carry += tot;
                __syncthreads();
            }
        }
        uint8_t *tile = region + (uint64_t)t * a.tb;
        const uint32_t n = i1 - i0;
        uint32_t wb[4]; // first slot of sections 8,4,2,1
        wb[0] = 0;
        wb[1] = sh.hist[G];
        wb[2] = sh.hist[2 * G];
        wb[3] = sh.hist[3 * G];
        uint32_t cnt[4];
        cnt[0] = wb[1];
        cnt[1] = wb[2] - wb[1];
        cnt[2] = wb[3] - wb[2];
        cnt[3] = n - wb[3];
        uint32_t off[4]; // byte offset of each section's first record
        off[0] = kHdr;
        off[1] = off[0] + 64u * cnt[0];
        off[2] = off[1] + 32u * cnt[1];
        off[3] = off[2] + 16u * cnt[2];
        const uint32_t se_off = off[3] + 8u * cnt[3];
        // thread g walks column g's rows in order: bucket ranks follow the row
        for (int g = tid; g < G; g += kT) {
            uint32_t run[4] = {0, 0, 0, 0};
            for (int r = ra; r <= rb; r++) {
                const uint32_t i = (uint32_t)r * G + g;
                if (i < i0 || i >= i1)
                    continue;
                const int nn = n0 + r;
                const uint64_t rs = (uint64_t)nn * a.nS + (g >> 5);
                const uint32_t p0 = wmap[2 * rs], p1 = wmap[2 * rs + 1];
                const WidthMasks wm = width_masks(p0, p1, min(32, G - 32 * (g >> 5)));
                const int c = width_code(p0, p1, g & 31);
                const int sec = 3 - c;
                const uint32_t rk = pick4(run, sec);
                run[0] += sec == 0;
                run[1] += sec == 1;
                run[2] += sec == 2;
                run[3] += sec == 3;
                const uint32_t slot = sh.hist[sec * G + g] + rk;
                const uint64_t src = (uint64_t)rowoff[nn] * kRowPad + sloff[rs] + group_offset_in_slice(wm, c, g & 31);
                const uint32_t dst = pick4(off, sec) + (slot - pick4(wb, sec)) * (8u << c);
                const uint32_t *s32 = reinterpret_cast<const uint32_t *>(codes + src);
                uint32_t *d32 = reinterpret_cast<uint32_t *>(tile + dst);
                for (int d = 0; d < (2 << c); d++)
                    d32[d] = s32[d];
                const uint32_t e = (uint32_t)g * (uint32_t)NR + (uint32_t)(r - ra);
                reinterpret_cast<uint32_t *>(tile + se_off)[slot] = (uint32_t)scales[(uint64_t)nn * G + g] | (e << 16);
            }
        }
        if (tid == 0) {
            uint32_t *h = reinterpret_cast<uint32_t *>(tile);
            h[0] = cnt[0];
            h[1] = cnt[1];
            h[2] = cnt[2];
            h[3] = cnt[3];
            h[4] = (uint32_t)ra;
            h[5] = (uint32_t)NR;
            h[6] = i0 - (uint32_t)ra * G;         // first column of row ra in this tile
            h[7] = i1 - 1 - (uint32_t)rb * G + 1; // one past the last column of row rb
            h[8] = NR == 1 ? 0u : (uint32_t)((0x100000000ull + (uint64_t)NR - 1) / (uint64_t)NR);
            h[9] = t + 1 < ntiles ? (uint32_t)kHdr + sh.tcum[t + 2] - sh.tcum[t + 1] : 0u; // next tile's bytes
            h[10] = n;
            h[11] = se_off;
            h[12] = se_off + 4u * n; // this tile's bytes
            h[13] = t;
            h[14] = ntiles;
            h[15] = VBQ_PLAN_MAGIC;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// The planned GEMV kernel.

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (m0 = lds_base, wave-uniform).  Written as asm so the compiler does not tie
// later LDS reads to it; completion is awaited explicitly (wait_vm0) before the
// barrier that publishes a tile.  The s_nop separates the m0 write from the load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

__device__ __forceinline__ void wait_vm0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));

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

// Copy `bytes` from global memory to LDS in 1 KiB chunks (16 bytes per lane,
// the tail masked per 16 bytes): this wave issues chunks first, first + step, ...
__device__ __forceinline__ void copy_chunks(const uint8_t *src, uint32_t dst, uint32_t bytes, int first, int step)
{
    const uint32_t lane16 = (threadIdx.x & 63) * 16u;
    for (uint32_t j = (uint32_t)first; j * 1024u < bytes; j += (uint32_t)step) {
        const uint32_t off = j * 1024u + lane16;
        if (off < bytes)
            dma16(src + off, dst + j * 1024u);
    }
}

// Kernel arguments.  The argument segment is read from memory at every
// launch and is not kept in the caches between launches, so each round of
// dependent argument loads costs a full memory round trip before a workgroup
// can start.  A workgroup therefore finds everything it needs in ONE 64-byte
// record, picked by blockIdx.y (the matrix of a shared launch), which it reads
// with a single scalar load.  Launch-wide fields are repeated in every record.
struct PRec {
    const uint8_t *plan;  // this matrix's plan
    void *y;              // its outputs (this launch's first token)
    const uint16_t *x;    // activations (this launch's first token)
    uint32_t region;      // bytes per row block of the plan
    int32_t N, ldy, rows; // rows per block of this matrix
    int32_t ldx;
    uint32_t first;       // bytes of tile 0 to copy (launch-wide maximum)
    int32_t ps;           // partial sums per token per ring slot (launch-wide)
    int32_t rows_max;     // output staging stride in LDS (launch-wide)
    uint32_t g_yt_tb;     // G | yt << 16 | (tile stride / 1 KiB) << 24
    int32_t wgs;          // row blocks of this matrix (workgroups with blockIdx.x < wgs work)
};
static_assert(sizeof(PRec) == 64, "one record is one 64-byte line");

// The launch that follows on the stream: where each of its workgroups starts
// reading.  Plans do not depend on the activations, so a workgroup of this
// launch fetches, during its last tile, the first tile of the workgroup with
// the same linear index there, which then finds it in the caches instead of
// waiting for HBM.  Read once, late, by the copying waves.
struct PWarm {
    const uint8_t *plan[kMaxMats]; // null: no such matrix
    uint32_t region[kMaxMats];     // bytes per row block
    uint16_t first16[kMaxMats];    // bytes of tile 0 / 16
    uint16_t wgs[kMaxMats];        // row blocks
};
static_assert(sizeof(PWarm) == 64, "the warming line is one 64-byte line");

struct PArgs {
    PRec rec[kMaxMats];
    PWarm warm;
};

struct PLayout {
    uint32_t x, ring, psum, ybuf, ctr, best, total;
};

__host__ __device__ inline uint32_t p_take(uint32_t &o, uint32_t bytes)
{
    const uint32_t r = o;
    o += (bytes + 15u) & ~15u;
    return r;
}

// LDS carve-up, computed identically on the host (size) and the device.
__host__ __device__ inline PLayout p_layout(int MT, int G, int rows, int tb, int ps)
{
    PLayout l;
    uint32_t o = 0;
    l.x = p_take(o, (uint32_t)(MT * G * kXRec * 4));
    l.ring = p_take(o, 2u * (uint32_t)tb);
    l.psum = p_take(o, 2u * (uint32_t)(MT * ps) * 4u);
    l.ybuf = p_take(o, (uint32_t)(MT * rows) * 4u);
    l.ctr = p_take(o, 2u * 4u); // pass counters of the two ring slots
    l.best = p_take(o, 2u * 8u); // argmax output: the best (value, row) key per token
    l.total = o;
    return l;
}

// x records (kXRec dwords per group; the 36-dword stride spreads the records
// of different columns over the LDS banks): the fp16 pairs (x_p, x_{p+32}),
// then the negated corrections -C_b for the widths 1, 2, 4, 8, where
// C_b = sum_p 2^(10-pos_b(p)) (x_p + x_{p+32}) + (2^b-1)/2 sum_j x_j.
// Item = (token, group, quarter q): pairs 4q..4q+3; the 8 items of a group are
// 8 adjacent lanes.  Loads and stores are separate so the loads go out with
// the first tile's copy.
// Prologue split: the first kCT threads copy tile 0 (a few waves issue the
// whole LDS-DMA copy), the other kXT threads stage x, which is the longer of
// the two (every workgroup reads the same activations, and each quarter-group
// item costs about 50 VALU instructions).
constexpr int kCT = 4 * 64;
constexpr int kXT = kT - kCT;

template <int MT>
struct XRegs {
    static constexpr int kPer = (MT * kMaxG * 8 + kXT - 1) / kXT;
    uint32_t lo0[kPer], lo1[kPer], hi0[kPer], hi1[kPer];
};

template <int MT>
__device__ __forceinline__ void x_load(const uint16_t *x, int ldx, int G, XRegs<MT> &xs)
{
    const int tid = threadIdx.x - kCT;
    const int items = MT * G * 8;
    const bool vec = (ldx % 4) == 0 && ((uintptr_t)x % 8) == 0;
#pragma unroll
    for (int k = 0; k < XRegs<MT>::kPer; k++) {
        const int i = tid + k * kXT;
        xs.lo0[k] = xs.lo1[k] = xs.hi0[k] = xs.hi1[k] = 0u;
        if (i < items) {
            const int q = i & 7, g = (i >> 3) % G, m = (i >> 3) / G;
            const uint16_t *p = x + (uint64_t)m * ldx + 64ull * g + 4 * q;
            if (vec) {
                const uint2 va = *reinterpret_cast<const uint2 *>(p);
                const uint2 vb = *reinterpret_cast<const uint2 *>(p + 32);
                xs.lo0[k] = va.x;
                xs.lo1[k] = va.y;
                xs.hi0[k] = vb.x;
                xs.hi1[k] = vb.y;
            } else {
                xs.lo0[k] = p[0] | ((uint32_t)p[1] << 16);
                xs.lo1[k] = p[2] | ((uint32_t)p[3] << 16);
                xs.hi0[k] = p[32] | ((uint32_t)p[33] << 16);
                xs.hi1[k] = p[34] | ((uint32_t)p[35] << 16);
            }
        }
    }
}

// v from another lane of the same DPP row (ctrl: a DPP control code).
template <int kCtrl>
__device__ __forceinline__ float dpp_f(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, 0xf, 0xf, false));
}

// Sum of v over each aligned group of L lanes (L = 8, 16, 32, 64), the same
// value in every lane of the group, in a fixed order: pairs and quads (DPP
// quad permutations), then the two quads of each 8 lanes (row_half_mirror:
// once every lane of a quad holds the quad's sum, the mirrored lane holds the
// other quad's), then the two halves of each 16-lane row (row_mirror), then
// across rows.  Lane moves inside a row cost no LDS traffic.
template <int L>
__device__ __forceinline__ float group_sum(float v)
{
    v += dpp_f<0xB1>(v);  // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);  // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v); // row_half_mirror
    if (L >= 16)
        v += dpp_f<0x140>(v); // row_mirror
    if (L >= 32)
        v += __shfl_xor(v, 16, 64);
    if (L >= 64)
        v += __shfl_xor(v, 32, 64);
    return v;
}

template <int MT>
__device__ __forceinline__ void x_store(int G, const XRegs<MT> &xs, uint32_t *xrec)
{
    const int tid = threadIdx.x - kCT;
    const int items = MT * G * 8;
#pragma unroll
    for (int k = 0; k < XRegs<MT>::kPer; k++) {
        const int i = tid + k * kXT;
        if (i >= items) // whole groups of 8 lanes drop out together
            break;
        const int q = i & 7, g = (i >> 3) % G, m = (i >> 3) / G;
        U4 o;
        o.v[0] = __builtin_amdgcn_perm(xs.hi0[k], xs.lo0[k], 0x05040100u); // (x_p, x_{p+32})
        o.v[1] = __builtin_amdgcn_perm(xs.hi0[k], xs.lo0[k], 0x07060302u);
        o.v[2] = __builtin_amdgcn_perm(xs.hi1[k], xs.lo1[k], 0x05040100u);
        o.v[3] = __builtin_amdgcn_perm(xs.hi1[k], xs.lo1[k], 0x07060302u);
        uint32_t *xr = xrec + ((uint32_t)m * G + g) * kXRec;
        *reinterpret_cast<U4 *>(xr + 4 * q) = o;
        float X = 0.f, c1 = 0.f, c2 = 0.f, c4 = 0.f;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int t = 4 * q + j; // pair index in the group
            const float sp = dot2(o.v[j], 0x3c003c00u, 0.f); // x_t + x_{t+32}, exact in fp32
            X += sp;
            c1 = fmaf((float)(1 << (10 - pair_pos<1>(t & 15))), sp, c1);
            c2 = fmaf((float)(1 << (10 - pair_pos<2>(t & 7))), sp, c2);
            c4 = fmaf((float)(1 << (10 - pair_pos<4>(t & 3))), sp, c4);
        }
        // fixed-order tree over the 8 quarters of the group
        X = group_sum<8>(X);
        c1 = group_sum<8>(c1);
        c2 = group_sum<8>(c2);
        c4 = group_sum<8>(c4);
        if (q == 0)
            *reinterpret_cast<U4 *>(xr + 32) =
                U4{{__float_as_uint(-fmaf(0.5f, X, c1)), __float_as_uint(-fmaf(1.5f, X, c2)),
                    __float_as_uint(-fmaf(7.5f, X, c4)), __float_as_uint(-fmaf(127.5f, X, 1024.f * X))}};
    }
}

// Header fields of one tile, kept in registers.
struct Tile {
    uint32_t cnt[4]; // groups per section (widths 8,4,2,1)
    uint32_t ra, nr, g_first, g_end, inv_nr, next, n, se_off;
};

// One lane reads the header (48 bytes instead of 3 KiB of LDS traffic per
// wave) and the fields are broadcast to the wave.  (Reading it from memory
// through the scalar cache instead would share the lgkmcnt counter with the
// passes' LDS reads and make them wait for that load.)
__device__ __forceinline__ Tile read_tile(const uint8_t *t)
{
    uint4 a = make_uint4(0u, 0u, 0u, 0u), b = a, c = a;
    if ((threadIdx.x & 63) == 0) {
        a = *reinterpret_cast<const uint4 *>(t);
        b = *reinterpret_cast<const uint4 *>(t + 16);
        c = *reinterpret_cast<const uint4 *>(t + 32);
    }
#define VBQ_BCAST(v) v = (uint32_t)__builtin_amdgcn_readfirstlane((int)v)
    VBQ_BCAST(a.x); VBQ_BCAST(a.y); VBQ_BCAST(a.z); VBQ_BCAST(a.w);
    VBQ_BCAST(b.x); VBQ_BCAST(b.y); VBQ_BCAST(b.z); VBQ_BCAST(b.w);
    VBQ_BCAST(c.x); VBQ_BCAST(c.y); VBQ_BCAST(c.z); VBQ_BCAST(c.w);
#undef VBQ_BCAST
    Tile h;
    h.cnt[0] = a.x;
    h.cnt[1] = a.y;
    h.cnt[2] = a.z;
    h.cnt[3] = a.w;
    h.ra = b.x;
    h.nr = b.y;
    h.g_first = b.z;
    h.g_end = b.w;
    h.inv_nr = c.x;
    h.next = c.y;
    h.n = c.z;
    h.se_off = c.w;
    return h;
}

// One pass: slots j = 64 * q + lane of the section of width B.
template <int B, int MT>
__device__ __forceinline__ void plan_pass(int q, uint32_t cnt, uint32_t wb, uint32_t code_off, const uint8_t *tile,
                                          const Tile &h, int G, int ps, const uint32_t *xrec, float *psum)
{
    constexpr int C = B == 1 ? 0 : B == 2 ? 1 : B == 4 ? 2 : 3;
    const uint32_t j = 64u * (uint32_t)q + (threadIdx.x & 63);
    if (j >= cnt)
        return;
    const uint32_t se = reinterpret_cast<const uint32_t *>(tile + h.se_off)[wb + j];
    uint32_t w[2 * B];
    const U2 *src = reinterpret_cast<const U2 *>(tile + code_off + j * (8u * B));
#pragma unroll
    for (int k = 0; k < B; k++) {
        const U2 v = src[k];
        w[2 * k] = v.v[0];
        w[2 * k + 1] = v.v[1];
    }
    uint32_t hp[32];
    unpack_pairs<B>(w, hp);
    const uint32_t e = se >> 16;
    const uint32_t xcol = h.nr == 1 ? e : __umulhi(e, h.inv_nr);
    const float s = __half2float(__ushort_as_half((uint16_t)(se & 0xffffu)));
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const uint32_t *xr = xrec + ((uint32_t)m * G + xcol) * kXRec;
        // two chains, the first starting from -C_b: pairs 0..15, then 16..31
        float acc0 = __uint_as_float(xr[32 + C]), acc1 = 0.f;
#pragma unroll
        for (int k = 0; k < 8; k++) {
            const U4 xa = *reinterpret_cast<const U4 *>(xr + 4 * k);
#pragma unroll
            for (int t = 0; t < 4; t++) {
                if (k < 4)
                    acc0 = dot2(hp[4 * k + t], xa.v[t], acc0);
                else
                    acc1 = dot2(hp[4 * k + t], xa.v[t], acc1);
            }
        }
        psum[m * ps + e] = s * (acc0 + acc1);
    }
}

// Lanes that sum one row: more for longer rows, so that a tile's row sums
// stay short next to its passes (a row of G partials is G / lanes loads deep).
__device__ __forceinline__ int sum_lanes(int G) { return G > 256 ? 64 : G > 128 ? 32 : G > 64 ? 16 : 8; }

// Row-sum items of a tile with nr rows.
__device__ __forceinline__ int sum_items(int nr, int G) { return (nr * sum_lanes(G) + 63) / 64; }

// Where finished rows go.
// Output modes, a template parameter of the kernel (a plain GEMV carries no
// code of the others).  kRows: finished rows are stored as fp32 or fp16 (yt).
// kArgmax: instead of storing rows, keep per token the largest (value,
// smallest row) as one 64-bit key in LDS (see argmax_key).  kSwiglu: rows 2i
// and 2i+1 are the gate and up rows of output i; finished rows stay in the
// LDS staging and the workgroup writes silu(gate) * up (type yt) for its
// pairs at the end.
constexpr int kRows = 0;
constexpr int kArgmax = 1;
constexpr int kSwiglu = 2;

struct YOut {
    void *y;
    int ldy, n0, yt;
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

// Row-sum item t of a tile: rows (64 / L) t .. of the tile, L = sum_lanes(G)
// lanes per row.  The partials of row j sit at column * nr + j for the tile's
// columns of that row; lane q sums columns q, q + L, ... (four interleaved
// chains), the L lanes combine in a fixed order (group_sum), and the row's sum from
// earlier tiles (ybuf, tiles in order) is added.  A row that ends in this
// tile is written to y; only a row that continues into the next tile stays in
// ybuf.
template <int MT, int OM, int L>
__device__ __forceinline__ void rowsum_item_l(int t, const Tile &h, int G, int ps, int rows, const float *psum,
                                              float *ybuf, const YOut &yo)
{
    const int lane = threadIdx.x & 63;
    constexpr int per = 64 / L;
    const int j = per * t + lane / L, q = lane & (L - 1);
    const int nr = (int)h.nr;
    const int lo = j == 0 ? (int)h.g_first : 0, hi = j == nr - 1 ? (int)h.g_end : G;
    const bool done = j < nr - 1 || (int)h.g_end == G || h.next == 0;
#pragma unroll
    for (int m = 0; m < MT; m++) {
        float v = 0.f;
        if (j < nr) {
            const float *p = psum + m * ps + j;
            float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
            int g = lo + q;
            const int step = L * nr; // column g + L of the row sits L * nr further
            const float *pg = p + g * nr;
            for (; g + 3 * L < hi; g += 4 * L, pg += 4 * step) {
                a0 += pg[0];
                a1 += pg[step];
                a2 += pg[2 * step];
                a3 += pg[3 * step];
            }
            for (; g < hi; g += L, pg += step)
                a0 += pg[0];
            v = (a0 + a1) + (a2 + a3);
        }
        v = group_sum<L>(v);
        if (q == 0 && j < nr) {
            const int r = (int)h.ra + j;
            const float tot = ybuf[m * rows + r] + v;
            if (done) {
                const uint64_t o = (uint64_t)m * yo.ldy + yo.n0 + r;
                if constexpr (OM == kArgmax)
                    atomicMax(yo.best + m, argmax_key(tot, (uint32_t)(yo.n0 + r)));
                else if constexpr (OM == kSwiglu)
                    ybuf[m * rows + r] = tot;
                else if (yo.yt == VBQ_F16)
                    reinterpret_cast<__half *>(yo.y)[o] = __float2half_rn(tot);
                else
                    reinterpret_cast<float *>(yo.y)[o] = tot;
            } else {
                ybuf[m * rows + r] = tot;
            }
        }
    }
}

template <int MT, int OM>
__device__ __forceinline__ void rowsum_item(int t, const Tile &h, int G, int ps, int rows, const float *psum,
                                            float *ybuf, const YOut &yo)
{
    switch (sum_lanes(G)) {
    case 8: rowsum_item_l<MT, OM, 8>(t, h, G, ps, rows, psum, ybuf, yo); break;
    case 16: rowsum_item_l<MT, OM, 16>(t, h, G, ps, rows, psum, ybuf, yo); break;
    case 32: rowsum_item_l<MT, OM, 32>(t, h, G, ps, rows, psum, ybuf, yo); break;
    default: rowsum_item_l<MT, OM, 64>(t, h, G, ps, rows, psum, ybuf, yo); break;
    }
}

// Merge this workgroup's keys into the call's (agent-scope atomics on the
// workspace); the last workgroup of the launch (a ticket counter) decodes the
// keys of its tokens into index and value and clears keys and counter for the
// next call.  tok0: the launch's first token.
template <int MT>
__device__ void argmax_finish(vbq_argmax_ws *ws, int tok0, const unsigned long long *best)
{
#pragma unroll
    for (int m = 0; m < MT; m++)
        __hip_atomic_fetch_max(&ws->key[tok0 + m], best[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t total = gridDim.x * gridDim.y;
    const uint32_t ticket = __hip_atomic_fetch_add(&ws->count, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (ticket != total - 1)
        return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const unsigned long long k =
            __hip_atomic_load(&ws->key[tok0 + m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint32_t ord = (uint32_t)(k >> 32);
        const uint32_t u = (ord & 0x80000000u) ? (ord & 0x7fffffffu) : ~ord;
        ws->index[tok0 + m] = (int32_t)(~(uint32_t)k);
        ws->value[tok0 + m] = __uint_as_float(u);
        __hip_atomic_store(&ws->key[tok0 + m], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(&ws->count, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MT, int OM>
__global__ __launch_bounds__(kT) void k_gemv_plan(PArgs /* read through kernarg_line */)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this workgroup's record (matrix blockIdx.y of the launch), in one load
    const u32x16 a = kernarg_line((uint32_t)blockIdx.y * (uint32_t)sizeof(PRec));
    if ((int)blockIdx.x >= (int)a[15])
        return; // the launch spans the largest matrix; a smaller one has fewer blocks
    const uint8_t *plan = (const uint8_t *)u64_ptr(a[0], a[1]);
    void *const yptr = (void *)u64_ptr(a[2], a[3]);
    const uint16_t *xptr = (const uint16_t *)u64_ptr(a[4], a[5]);
    const uint32_t region_bytes = a[6];
    const int Nm = (int)a[7], ldy = (int)a[8], mrows = (int)a[9], ldx = (int)a[10];
    const uint32_t first = a[11];
    const int ps = (int)a[12], rows = (int)a[13];
    const int G = (int)(a[14] & 0xffffu), yt = (int)((a[14] >> 16) & 0xffu);
    const uint32_t tb = (a[14] >> 24) * 1024u;
    const int blk = (int)blockIdx.x;
    const int n0 = blk * mrows;
    const int R = min(mrows, Nm - n0);
    const PLayout L = p_layout(MT, G, rows, (int)tb, ps);
    uint32_t *xrec = reinterpret_cast<uint32_t *>(smem + L.x);
    float *psum = reinterpret_cast<float *>(smem + L.psum);
    float *ybuf = reinterpret_cast<float *>(smem + L.ybuf);
    const uint8_t *region = plan + (uint64_t)blk * region_bytes;
    const uint32_t ring = lds_addr(smem + L.ring);
    unsigned long long *best = reinterpret_cast<unsigned long long *>(smem + L.best);
    const YOut yo{yptr, ldy, n0, yt, best};
    const uint8_t *warm = nullptr; // set by the copying waves before the last tile's phase
    uint32_t warm_bytes = 0;

    // ---- tile 0 (copied by the first kCT threads) and the activations
    // (staged by the others), in flight together; each side waits only for
    // its own loads
    uint32_t *cnt = reinterpret_cast<uint32_t *>(smem + L.ctr);
    if (tid < kCT) {
        copy_chunks(region, ring, first, wave, kCT / 64);
        for (int i = tid; i < MT * R; i += kCT)
            ybuf[(i / R) * rows + i % R] = 0.f;
        if (tid == 0)
            cnt[0] = 0u;
        if (tid < MT)
            best[tid] = 0ull;
        wait_vm0();
    } else {
        XRegs<MT> xs;
        x_load<MT>(xptr, ldx, G, xs);
        x_store<MT>(G, xs, xrec);
    }
    __syncthreads();

    // ---- tile k sits in ring slot k & 1: wave 0 copies tile k+1 into the
    // other slot while waves 1.. run the passes of tile k; then all waves sum
    // the rows of tile k-1 (partials in psum slot (k-1) & 1).
    Tile prev{};
    int k = 0;
    for (;; k++) {
        const int slot = k & 1;
        const uint8_t *tile = smem + L.ring + (uint32_t)slot * tb;
        const Tile h = read_tile(tile);
        float *ps_k = psum + slot * (MT * ps);
        if (wave < kCopyWaves) {
            if (tid == 0)
                cnt[slot ^ 1] = 0u; // pass counter of tile k+1 (its last users left tile k-1's phase)
            if (!h.next) {
                // last tile: the next launch's workgroup with this linear
                // index, whose first tile goes into the free slot (awaited at
                // the very end)
                const u32x16 w = kernarg_line((uint32_t)(kMaxMats * sizeof(PRec)));
                uint32_t gx = 0;
#pragma unroll
                for (int i = 0; i < kMaxMats; i++)
                    gx = max(gx, w[14 + i / 2] >> (16 * (i & 1)) & 0xffffu);
                const uint32_t lin = blockIdx.y * gridDim.x + blockIdx.x;
                const uint32_t bx = gx ? lin % gx : 0u, by = gx ? lin / gx : (uint32_t)kMaxMats;
#pragma unroll
                for (int i = 0; i < kMaxMats; i++) {
                    const uint32_t wgs_i = w[14 + i / 2] >> (16 * (i & 1)) & 0xffffu;
                    const uint32_t first_i = (w[12 + i / 2] >> (16 * (i & 1)) & 0xffffu) * 16u;
                    const uint8_t *p_i = (const uint8_t *)u64_ptr(w[2 * i], w[2 * i + 1]);
                    const bool mine = by == (uint32_t)i && bx < wgs_i && p_i != nullptr;
                    warm = mine ? p_i + (uint64_t)bx * w[8 + i] : warm;
                    warm_bytes = mine ? min(first_i, tb) : warm_bytes;
                }
            }
            // tile k+1, or after the last tile the warming copy
            copy_chunks(h.next ? region + (uint64_t)(k + 1) * tb : warm, ring + (uint32_t)(slot ^ 1) * tb,
                        h.next ? h.next : warm_bytes, wave, kCopyWaves);
        } else {
            const int np0 = (int)((h.cnt[0] + 63) >> 6), np1 = (int)((h.cnt[1] + 63) >> 6);
            const int np2 = (int)((h.cnt[2] + 63) >> 6), np3 = (int)((h.cnt[3] + 63) >> 6);
            const int pb1 = np0, pb2 = pb1 + np1, pb3 = pb2 + np2, np = pb3 + np3;
            const uint32_t wb1 = h.cnt[0], wb2 = wb1 + h.cnt[1], wb3 = wb2 + h.cnt[2];
            const uint32_t off1 = kHdr + 64u * h.cnt[0], off2 = off1 + 32u * h.cnt[1], off3 = off2 + 16u * h.cnt[2];
            // worker w runs pass w first; later passes come from an LDS counter,
            // each asked for before the current pass runs so that the atomic's
            // latency hides behind it
            constexpr int nw = kW - kCopyWaves;
            uint32_t nextp = 0;
            for (int p = wave - kCopyWaves; p < np; p = __builtin_amdgcn_readfirstlane((int)nextp)) {
                if ((tid & 63) == 0)
                    nextp = nw + atomicAdd(cnt + slot, 1u);
                if (p < pb1)
                    plan_pass<8, MT>(p, h.cnt[0], 0u, kHdr, tile, h, G, ps, xrec, ps_k);
                else if (p < pb2)
                    plan_pass<4, MT>(p - pb1, h.cnt[1], wb1, off1, tile, h, G, ps, xrec, ps_k);
                else if (p < pb3)
                    plan_pass<2, MT>(p - pb2, h.cnt[2], wb2, off2, tile, h, G, ps, xrec, ps_k);
                else
                    plan_pass<1, MT>(p - pb3, h.cnt[3], wb3, off3, tile, h, G, ps, xrec, ps_k);
            }
        }
        if (k > 0) {
            const int nsum = sum_items((int)prev.nr, G);
            for (int t = (wave + kW - kCopyWaves) % kW; t < nsum; t += kW) // copying waves take the last shares
                rowsum_item<MT, OM>(t, prev, G, ps, rows, psum + (slot ^ 1) * (MT * ps), ybuf, yo);
        }
        if (h.next)
            wait_vm0(); // copy waves: the copy of tile k+1
        __syncthreads();
        prev = h;
        if (!h.next)
            break;
    }
    // ---- rows of the last tile (partials in psum slot k & 1); every row ends here
    {
        const int nsum = sum_items((int)prev.nr, G);
        for (int t = (wave + kW - kCopyWaves) % kW; t < nsum; t += kW) // copying waves take the last shares
            rowsum_item<MT, OM>(t, prev, G, ps, rows, psum + (k & 1) * (MT * ps), ybuf, yo);
    }
    // the warming copy lands in LDS: it must finish before the workgroup's LDS
    // is released (the other waves leave without waiting for their stores)
    if (wave < kCopyWaves && warm_bytes)
        wait_vm0();
    if constexpr (OM == kArgmax) {
        __syncthreads(); // every finished row's key is in best[]
        if (tid == 0)
            argmax_finish<MT>(reinterpret_cast<vbq_argmax_ws *>(yptr), ldy, best);
    } else if constexpr (OM == kSwiglu) {
        __syncthreads(); // every row of the block is in ybuf
        const int pairs = R / 2; // R is even: the block starts at an even row and N is even
        for (int i = tid; i < MT * pairs; i += kT) {
            const int m = i / pairs, p = i - m * pairs;
            const float g = ybuf[m * rows + 2 * p], u = ybuf[m * rows + 2 * p + 1];
            const float h = g / (1.0f + expf(-g)) * u; // silu(gate) * up
            const uint64_t o = (uint64_t)m * ldy + n0 / 2 + p;
            if (yt == VBQ_F16)
                reinterpret_cast<__half *>(yptr)[o] = __float2half_rn(h);
            else
                reinterpret_cast<float *>(yptr)[o] = h;
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

int plan_cus()
{
    static int cus = 0;
    if (!cus) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            cus = 256;
    }
    return cus;
}

constexpr uint32_t kLdsBudget = 160u * 1024u;

// Partial-sum capacity of a tile: groups (at least 12 bytes each) plus the
// columns of a first and a last row the tile only partly covers.
int psum_capacity(int tb, int G) { return (tb - kHdr) / 12 + 2 * G; }

vbq_status check_plan(const vbq_plan *P)
{
    if (!P || P->magic != VBQ_PLAN_MAGIC)
        return VBQ_ERR_LAYOUT;
    if (P->N < 1 || P->G < 1 || P->G > kMaxG || P->K != 64 * P->G || P->M < 1 || P->M > 2 || P->wgs < 1 ||
        P->rows < 1 || (int64_t)P->wgs * P->rows < P->N || (int64_t)(P->wgs - 1) * P->rows >= P->N ||
        P->wgs > 65535 || P->tiles > kMaxTiles || P->tile_bytes < 4096 || P->tile_bytes > kMaxTb ||
        P->tile_bytes % 1024 || P->tiles < 1 || P->first_bytes < kHdr || P->first_bytes > P->tile_bytes ||
        P->region_bytes != (uint64_t)P->tiles * (uint64_t)P->tile_bytes)
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
    a.tb = (uint32_t)P->tile_bytes;
    a.region = P->region_bytes;
    return a;
}

template <int MT, int OM>
vbq_status launch_plan_t(const PArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    static bool configured = false;
    if (!configured) {
        VBQ_TRY(hip_status(
            hipFuncSetAttribute((const void *)k_gemv_plan<MT, OM>, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBudget)));
        configured = true;
    }
    hipLaunchKernelGGL((k_gemv_plan<MT, OM>), dim3(grid), dim3(kT), lds, stream, a);
    return launch_status();
}

// One launch of m (1 or 2) tokens in output mode om.
vbq_status launch_plan(int m, int om, const PArgs &a, dim3 grid, uint32_t lds, hipStream_t stream)
{
    switch (om * 2 + (m - 1)) {
    case 0: return launch_plan_t<1, kRows>(a, grid, lds, stream);
    case 1: return launch_plan_t<2, kRows>(a, grid, lds, stream);
    case 2: return launch_plan_t<1, kArgmax>(a, grid, lds, stream);
    case 3: return launch_plan_t<2, kArgmax>(a, grid, lds, stream);
    case 4: return launch_plan_t<1, kSwiglu>(a, grid, lds, stream);
    default: return launch_plan_t<2, kSwiglu>(a, grid, lds, stream);
    }
}

} // namespace

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
    if (wgs <= 0)
        wgs = plan_cus();
    // an even row count whenever N is even, so that a row block never splits
    // the (gate, up) pairs of an interleaved SwiGLU matrix
    int rows = (N + wgs - 1) / wgs;
    if (N % 2 == 0 && rows % 2)
        rows++;
    wgs = (N + rows - 1) / rows;
    // the largest tile stride (1 KiB steps) whose launch fits the LDS budget;
    // two tokens per launch only while that keeps tiles of 16 KiB or more
    // (beyond, the x records of two tokens crowd out the tiles)
    int tb = 0;
    for (;;) {
        tb = 0;
        for (int cand = kMaxTb; cand >= 4096 && !tb; cand -= 1024) {
            const int ps = psum_capacity(cand, G);
            if (ps <= 65536 && p_layout(M, G, rows, cand, ps).total <= kLdsBudget)
                tb = cand;
        }
        if (M > 1 && tb < 16 * 1024) {
            M--;
            continue;
        }
        break;
    }
    if (!tb)
        return VBQ_ERR_SHAPE;
    vbq_plan p{};
    p.magic = VBQ_PLAN_MAGIC;
    p.N = N;
    p.K = (int)L->K;
    p.G = G;
    p.M = M;
    p.wgs = wgs;
    p.rows = rows;
    p.tile_bytes = tb;
    p.psum = psum_capacity(tb, G);
    p.lds_bytes = (int)p_layout(M, G, rows, tb, p.psum).total;
    // sizing pass: tiles per block region and the largest first tile
    VBQ_TRY(zero_words(ws, 16, stream));
    PrepArgs a = prep_args(L, blob, &p);
    a.plan = nullptr;
    a.sizes = (uint32_t *)ws;
    hipLaunchKernelGGL(k_prepare, dim3(wgs), dim3(kT), 0, stream, a);
    VBQ_TRY(launch_status());
    uint32_t h[4];
    VBQ_TRY(hip_status(hipMemcpyAsync(h, ws, 16, hipMemcpyDeviceToHost, stream)));
    VBQ_TRY(hip_status(hipStreamSynchronize(stream)));
    if (h[2] || h[0] < 1)
        return VBQ_ERR_SHAPE; // some block needs more tiles than a plan holds
    p.tiles = (int)h[0];
    p.first_bytes = (int)h[1];
    p.region_bytes = (uint64_t)p.tiles * (uint64_t)tb;
    p.total_bytes = (uint64_t)wgs * p.region_bytes;
    *P = p;
    return VBQ_OK;
}

vbq_status vbq_prepare(const vbq_plan *P, const vbq_layout *L, const void *blob, void *plan, hipStream_t stream)
{
    if (!blob || !plan)
        return VBQ_ERR_INVALID_ARG;
    VBQ_TRY(check_layout(L));
    VBQ_TRY(check_plan(P));
    if ((int)L->N != P->N || (int)L->K != P->K)
        return VBQ_ERR_SHAPE;
    if ((uintptr_t)blob % 256 || (uintptr_t)plan % 256)
        return VBQ_ERR_ALIGN;
    PrepArgs a = prep_args(L, blob, P);
    a.plan = (uint8_t *)plan;
    a.sizes = nullptr;
    hipLaunchKernelGGL(k_prepare, dim3(P->wgs), dim3(kT), 0, stream, a);
    return launch_status();
}

} // extern "C"

namespace {

// Checks one launch for up to P->M tokens (the plans' LDS carve-up holds that
// many) and fills its arguments; launches nothing.
vbq_status planned_args(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                        int tok0, PArgs *out, dim3 *grid_out, uint32_t *lds_out)
{
    if ((uintptr_t)x % 2)
        return VBQ_ERR_ALIGN;
    PArgs a{};
    int gx = 0, rows_max = 0;
    uint32_t first = 0;
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
        if (P->tile_bytes != P0->tile_bytes || P->psum != P0->psum)
            return VBQ_ERR_SHAPE; // one launch needs one LDS carve-up
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
        r.wgs = P->wgs;
        gx = std::max(gx, P->wgs);
        first = std::max(first, (uint32_t)P->first_bytes);
        rows_max = std::max(rows_max, P->rows); // output staging stride: the plan with the most rows fits
    }
    const vbq_plan *P0 = items[0].P;
    const uint32_t lds = p_layout(M, P0->G, rows_max, P0->tile_bytes, P0->psum).total;
    if (lds > kLdsBudget)
        return VBQ_ERR_SHAPE;
    for (int i = 0; i < n; i++) {
        PRec &r = a.rec[i];
        r.first = first;
        r.ps = P0->psum;
        r.rows_max = rows_max;
        r.g_yt_tb = (uint32_t)P0->G | (uint32_t)yt << 16 | (uint32_t)(P0->tile_bytes / 1024) << 24;
    }
    *out = a;
    *grid_out = dim3((unsigned)gx, (unsigned)n);
    *lds_out = lds;
    return VBQ_OK;
}

// Fills a.warm from the items of the launch that follows (none: no warming).
void set_next(PArgs &a, const vbq_planned_item *next, int nnext)
{
    a.warm = PWarm{};
    for (int i = 0; next && i < nnext && i < kMaxMats; i++) {
        const vbq_plan *P = next[i].P;
        a.warm.plan[i] = (const uint8_t *)next[i].plan;
        a.warm.region[i] = (uint32_t)P->region_bytes;
        a.warm.first16[i] = (uint16_t)((P->first_bytes + 15) / 16);
        a.warm.wgs[i] = (uint16_t)P->wgs;
    }
}

// Tokens beyond what one launch holds run as further launches over the same
// plans; each token's arithmetic is the same in every launch shape.  Every
// launch is checked before the first is enqueued; with stream == nullptr and
// dry set, only the checks run.
vbq_status planned_shared(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                          hipStream_t stream, bool dry, const vbq_planned_item *next = nullptr, int nnext = 0)
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
            // a further token chunk re-reads the same plans; after the last
            // chunk comes the caller's next launch
            if (t0 + chunk < M)
                set_next(a, items, n);
            else
                set_next(a, next, nnext);
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

vbq_status vbq::planned_shared_launch(const vbq_planned_item *items, int n, int M, const uint16_t *x, int ldx,
                                      vbq_dtype yt, hipStream_t stream, const vbq_planned_item *next, int nnext)
{
    return planned_shared(items, n, M, x, ldx, yt, stream, false, next, nnext);
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
            set_next(a, nullptr, 0);
            a.rec[0].y = (uint8_t *)h + (uint64_t)t0 * (uint64_t)ldh * (uint64_t)esz;
            a.rec[0].ldy = ldh;
            if (pass == 1)
                VBQ_TRY(launch_plan(m, kSwiglu, a, grid, lds, stream));
        }
    return VBQ_OK;
}

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
    const int chunk = P->M;
    // the same checks and arguments as an fp32 planned GEMV writing to ws, then
    // the record is switched to the argmax output (y = ws, ldy = first token)
    const vbq_planned_item it{P, plan, ws, P->N};
    PArgs a;
    dim3 grid;
    uint32_t lds;
    for (int pass = 0; pass < 2; pass++)
        for (int t0 = 0; t0 < M; t0 += chunk) {
            const int m = std::min(chunk, M - t0);
            VBQ_TRY(planned_args(&it, 1, m, x, ldx, VBQ_F32, t0, &a, &grid, &lds));
            set_next(a, nullptr, 0);
            a.rec[0].y = ws;
            a.rec[0].ldy = t0;
            if (pass == 1)
                VBQ_TRY(launch_plan(m, kArgmax, a, grid, lds, stream));
        }
    return VBQ_OK;
}

} // extern "C"
