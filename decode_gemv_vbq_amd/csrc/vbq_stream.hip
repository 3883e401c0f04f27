// Streaming GEMV over the VBQ1 layout for M = 1..2 tokens (gfx950).
//
// The decode path of "Variable Bit-width Quantization" (mlsanity.com page,
// Abstract): every contiguous group of 64 weights carries its own width in
// {1,2,4,8} and a scale, and decode multiplies by the dequantized weights
// without materialising them.  Decode is bound by HBM bandwidth, so this
// kernel is organised around one continuous stream of packed bytes per CU:
//
//  * One 1024-thread workgroup per CU owns a contiguous block of rows.  Its
//    rows' metadata (row offsets, slice offsets, width bit planes) and the
//    activations are read once at the start; x is kept in LDS as fp16 pairs
//    (x_p, x_{p+32}) per group plus four per-width correction constants.
//  * The block is cut into sub-units of whole rows holding at most 32 KiB of
//    code bytes (less when K is long).  A sub-unit's code bytes and scales are
//    contiguous in HBM, so they are copied straight into a two-slot LDS ring
//    with global_load_lds_dwordx4 (1 KiB per wave instruction, no VGPRs) while
//    the previous sub-unit computes: HBM sees a steady stream.  A block that
//    fits both slots is a single sub-unit (one table, no second round).
//  * Inside a sub-unit the groups are listed per width in a slot table, so a
//    wavefront always runs 64 groups of ONE width (no divergence between the
//    1/2/4/8-bit paths); the 16 waves take passes from an LDS counter.
//    Slots of a width are ordered (group half, slice, row, rank): a 16-lane
//    LDS phase then reads the x records of one 16-column window (equal columns
//    broadcast, distinct ones sit in distinct banks) except where the window
//    changes.
//  * Lane = one group: code words from LDS become fp16 pairs 2^(10-pos) + q
//    with one v_and_or_b32 each (8-bit: v_perm_b32), v_dot2_f32_f16 multiplies
//    two weights per instruction into fp32, and the group result is
//        s * (acc - C_b(g)),  C_b(g) = sum_p magic_p (x_p + x_{p+32}) + (2^b-1)/2 sum_j x_j.
//  * Partials land in LDS in natural (row, group) order and each row is
//    summed by 16 lanes in a fixed order: results do not depend on timing.
#include <algorithm>

#include "vbq_common.h"
#include "vbq_host.h"
#include "vbq_unpack.h"

using namespace vbq;

namespace {

constexpr int kT = 1024;                  // threads per workgroup (one per CU)
constexpr int kW = kT / 64;               // waves per workgroup
constexpr int kMaxCap = kT * 32;          // code bytes of one sub-unit, at most
constexpr int kMaxRS = kT / 8;            // row-slices of one sub-unit (8 lanes per row in the row phase)
constexpr int kRing = 2;                  // sub-units resident: one computing, one in flight
constexpr int kMaxSlots = kMaxRS * 32 + 4 * 64;   // slot table incl. per-width pass padding
constexpr int kMetaRS = kT;               // row-slices of metadata per workgroup (one load round each)
constexpr int kXRec = 36;                 // dwords per x record: 32 pairs + 4 constants
constexpr int kInfo = 16;                 // dwords per row-slice descriptor
constexpr int kPsum = kMaxRS * 32;        // partials per token

// Scale bytes of a sub-unit (+ 16-byte alignment slack).  The ring holds the
// code areas of its slots back to back, then their scale areas back to back,
// so that all slots together can serve as one double-size sub-unit.
__host__ __device__ constexpr uint32_t scale_area(int cap) { return (uint32_t)(cap / 4 + 128); }
__host__ __device__ constexpr uint32_t ring_bytes(int cap) { return (uint32_t)kRing * ((uint32_t)cap + scale_area(cap)); }

constexpr int kMaxMats = 4; // matrices sharing x in one launch

// One matrix of a launch: its blob, outputs and first workgroup.
struct SMat {
    const uint8_t *blob;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    void *y;
    int N, ldy, wg0;
};

struct SArgs {
    // the matrix of this workgroup, filled from mats[] at kernel start
    const uint8_t *blob;
    uint64_t off_row_off, off_slice_off, off_wmap, off_scales, off_codes;
    void *y;
    int N, ldy;
    // shared by all matrices of the launch (same K)
    int G, nS, M;
    const uint16_t *x;
    int ldx, yt;
    int rows;   // rows per workgroup
    int cap;    // code bytes per sub-unit (multiple of 1024, 8192..kMaxCap)
    int inv_nS; // ceil(65536 / nS): i / nS == (i * inv_nS) >> 16 for i < kMaxRS
    int nmat;
    SMat mats[kMaxMats];
};

// LDS carve-up, computed identically on the host (size) and the device.
struct SLayout {
    uint32_t x, rowoff, sloff, wmap, ring, info, hdr, table, psum, ybuf, total;
};

__host__ __device__ inline uint32_t s_take(uint32_t &o, uint32_t bytes)
{
    uint32_t r = o;
    o += (bytes + 15u) & ~15u;
    return r;
}

__host__ __device__ inline SLayout s_layout(int MT, int G, int rows, int nS, int cap)
{
    SLayout l;
    uint32_t o = 0;
    l.x = s_take(o, (uint32_t)(MT * G * kXRec * 4));
    l.rowoff = s_take(o, (uint32_t)((rows + 1) * 4));
    l.sloff = s_take(o, (uint32_t)(rows * nS * 4));
    l.wmap = s_take(o, (uint32_t)(rows * nS * 8));
    l.ring = s_take(o, ring_bytes(cap));
    l.info = s_take(o, (uint32_t)(2 * kMaxRS * kInfo * 4));
    l.hdr = s_take(o, 2 * 16 * 4);
    l.table = s_take(o, kMaxSlots * 4);
    l.psum = s_take(o, (uint32_t)(MT * kPsum * 4));
    l.ybuf = s_take(o, (uint32_t)(MT * rows * 4));
    l.total = o;
    return l;
}

__device__ __forceinline__ uint32_t lds_addr(const void *p)
{
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint8_t *)p;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16 * lane
// (m0 = lds_base, wave-uniform).  Written as asm so the compiler does not tie
// every later LDS read to it with a full vmcnt wait: completion is awaited
// explicitly (wait_vm) before the barrier that publishes a sub-unit.  The
// leading s_nop separates the compiler's m0 write from the LDS-DMA load.
__device__ __forceinline__ void dma16(const void *g, uint32_t lds_base)
{
    asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(g), "{m0}"(__builtin_amdgcn_readfirstlane(lds_base))
                 : "memory");
}

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

// Inclusive prefix sum over the 64 lanes (DPP row shifts and row broadcasts).
__device__ __forceinline__ int scan64(int v)
{
    v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false); // row_shr:1
    v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false); // row_shr:2
    v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false); // row_shr:4
    v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false); // row_shr:8
    v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false); // row_bcast:15
    v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false); // row_bcast:31
    return v;
}

struct Ctx {
    SArgs a;
    int n0, R;
    uint8_t *smem;
    SLayout L;
};

// First row after the sub-unit that starts at row ra: as many whole rows as
// fit `cap` code bytes and kMaxRS row-slices (at least one row).
__device__ __forceinline__ int next_end(const Ctx &c, int ra)
{
    if (ra >= c.R)
        return c.R;
    const uint32_t *rowoff = reinterpret_cast<const uint32_t *>(c.smem + c.L.rowoff);
    const int lane = threadIdx.x & 63;
    const int kmax = min(kMaxRS / c.a.nS, c.R - ra);
    const uint32_t base = rowoff[ra], cap = (uint32_t)c.a.cap;
    int n = 0;
#pragma unroll
    for (int h = 0; h < kMaxRS / 64; h++) {
        const int k = lane + 1 + 64 * h;
        const bool ok = k <= kmax && (rowoff[min(ra + k, c.R)] - base) * 128u <= cap;
        n += (int)__popcll(__ballot(ok)); // the condition is monotone in k
    }
    return ra + n;
}

// The copy of one sub-unit into a ring slot: code bytes [128*o0, 128*o1) of
// the codes section, then the scales of its rows, in 1 KiB chunks.  Chunk j
// belongs to wave (j + v) % kW; each wave issues its chunks in order, one at
// a time (issue_next), so the copy can be spread over the passes of the
// previous sub-unit instead of stalling every wave at once.
struct Copy {
    const uint8_t *gc, *gs;
    uint32_t dst, sdst, clen, slen;
    int nc, n, j; // code chunks, all chunks, this wave's next chunk
};

__device__ __forceinline__ uint32_t slot_codes(const Ctx &c, int slot) { return c.L.ring + (uint32_t)(slot * c.a.cap); }
__device__ __forceinline__ uint32_t slot_scales(const Ctx &c, int slot)
{
    return c.L.ring + (uint32_t)(kRing * c.a.cap) + (uint32_t)slot * scale_area(c.a.cap);
}

__device__ __forceinline__ Copy make_copy(const Ctx &c, uint32_t o0, uint32_t o1, int ra, int rb, int slot, int v)
{
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    Copy k;
    const uint64_t s0a = ((uint64_t)(c.n0 + ra) * c.a.G * 2u) & ~15ull;
    k.clen = (o1 - o0) * 128u;
    k.slen = (uint32_t)((uint64_t)(c.n0 + rb) * c.a.G * 2u - s0a);
    k.nc = (int)((k.clen + 1023u) >> 10);
    k.n = k.nc + (int)((k.slen + 1023u) >> 10);
    k.gc = c.a.blob + c.a.off_codes + (uint64_t)o0 * 128u;
    k.gs = c.a.blob + c.a.off_scales + s0a;
    k.dst = lds_addr(c.smem + slot_codes(c, slot));
    k.sdst = lds_addr(c.smem + slot_scales(c, slot));
    k.j = (wave - v % kW + kW) % kW;
    return k;
}

// Issues this wave's next chunk, if any; returns 1 if it issued one.
__device__ __forceinline__ int issue_next(const Ctx &c, Copy &k)
{
    if (k.j >= k.n)
        return 0;
    const int lane = threadIdx.x & 63;
    if (k.j < k.nc) {
        const uint32_t off = (uint32_t)k.j * 1024u + lane * 16u;
        if (off < k.clen)
            dma16(k.gc + off, k.dst + k.j * 1024u);
    } else {
        const uint32_t off = (uint32_t)(k.j - k.nc) * 1024u + lane * 16u;
        if (off < k.slen)
            dma16(k.gs + off, k.sdst + (k.j - k.nc) * 1024u);
    }
    k.j += kW;
    return 1;
}

__device__ __forceinline__ int issue_all(const Ctx &c, Copy &k)
{
    int cnt = 0;
    while (issue_next(c, k))
        cnt++;
    return cnt;
}

// Descriptors of the row-slices of rows [ra, rb), built by one wave (lane l
// holds row-slices 2l and 2l+1):
//   d0, d1    width bit planes
//   d2        row in sub-unit << 13 | first group column of the slice << 20
//   d3        valid groups
//   d4+3c     groups of width c (mask)
//   d5+3c     slot of the first half-0 group of width c | (slot of the first
//             half-1 group - half-0 groups of width c) << 16
//   d6+3c     record start / 8 + bucket start / 8 of width c
// Row-slices are numbered slice-major (slice * rows + row), so slots of width
// c are ordered (group half, slice, row, rank); each width starts on a 64-slot
// pass boundary.  Also resets the sub-unit's pass counter.
// Inputs of build_info for lane l's row-slices 2l and 2l+1 of the sub-unit
// starting at row ra: width planes, slice offset, row offset relative to row ra.
// ceil(65536 / n): (i * inv_rows(n)) >> 16 == i / n for 0 <= i < 128, 1 <= n <= 128.
__device__ __forceinline__ uint32_t inv_rows(int n) { return (65536u + (uint32_t)n - 1u) / (uint32_t)n; }

struct InfoIn {
    uint32_t p0[2], p1[2], slo[2], roff[2];
};

__device__ __forceinline__ void info_in_lds(const Ctx &c, int ra, int rb, InfoIn &in)
{
    const int lane = threadIdx.x & 63;
    const int nS = c.a.nS;
    const uint32_t *rowoff = reinterpret_cast<const uint32_t *>(c.smem + c.L.rowoff);
    const uint32_t *sloff = reinterpret_cast<const uint32_t *>(c.smem + c.L.sloff);
    const uint32_t *wmap = reinterpret_cast<const uint32_t *>(c.smem + c.L.wmap);
    const int Rs = rb - ra, nrs = Rs * nS;
    const uint32_t base0 = rowoff[ra], invR = inv_rows(Rs);
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int i = 2 * lane + j; // slice-major: i = slice * Rs + row
        const bool live = i < nrs;
        const int s = (int)(((uint32_t)i * invR) >> 16), r = i - s * Rs;
        const int w = live ? (ra + r) * nS + s : 0;
        in.p0[j] = live ? wmap[2 * w] : 0u;
        in.p1[j] = live ? wmap[2 * w + 1] : 0u;
        in.slo[j] = live ? sloff[w] : 0u;
        in.roff[j] = live ? rowoff[ra + r] - base0 : 0u;
    }
}

// Reorders InfoIn loaded in row-major row-slice order (lane l: row-slices 2l,
// 2l+1 of r * nS + s) into slice-major order for a sub-unit of Rs rows.
__device__ __forceinline__ void to_slice_major(InfoIn &in, int Rs, int nS)
{
    const int lane = threadIdx.x & 63;
    const uint32_t invR = inv_rows(Rs);
    InfoIn o;
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int i = 2 * lane + j;
        const int s = (int)(((uint32_t)i * invR) >> 16), r = i - s * Rs;
        const int src = min(r * nS + s, 127); // lanes past the sub-unit are masked later
        const int sl = src >> 1;
        const bool odd = src & 1;
        const uint32_t a0 = __shfl(in.p0[0], sl), a1 = __shfl(in.p0[1], sl);
        const uint32_t b0 = __shfl(in.p1[0], sl), b1 = __shfl(in.p1[1], sl);
        const uint32_t c0 = __shfl(in.slo[0], sl), c1 = __shfl(in.slo[1], sl);
        const uint32_t d0 = __shfl(in.roff[0], sl), d1 = __shfl(in.roff[1], sl);
        o.p0[j] = odd ? a1 : a0;
        o.p1[j] = odd ? b1 : b0;
        o.slo[j] = odd ? c1 : c0;
        o.roff[j] = odd ? d1 : d0;
    }
    in = o;
}

__device__ void build_info(const Ctx &c, int ra, int rb, int buf, const InfoIn &in)
{
    const int lane = threadIdx.x & 63;
    const int nS = c.a.nS, G = c.a.G;
    uint32_t *info = reinterpret_cast<uint32_t *>(c.smem + c.L.info) + buf * kMaxRS * kInfo;
    uint32_t *hdr = reinterpret_cast<uint32_t *>(c.smem + c.L.hdr) + buf * 16;
    const int Rs = rb - ra, nrs = Rs * nS;
    const uint32_t invR = inv_rows(Rs);
    uint32_t p0[2], p1[2], m[2][4], rec8[2];
    int ng[2], r[2], s[2], cnt[2][4], h0[2][4];
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int i = 2 * lane + j; // slice-major row-slice index
        const bool live = i < nrs;
        s[j] = (int)(((uint32_t)i * invR) >> 16);
        r[j] = i - s[j] * Rs;
        p0[j] = live ? in.p0[j] : 0u;
        p1[j] = live ? in.p1[j] : 0u;
        rec8[j] = live ? (in.roff[j] * 128u + in.slo[j]) >> 3 : 0u;
        ng[j] = live ? max(0, min(32, G - 32 * s[j])) : 0;
        const WidthMasks wm = width_masks(p0[j], p1[j], ng[j]);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            m[j][k] = wm.m[k];
            cnt[j][k] = __popc(wm.m[k]);
            h0[j][k] = __popc(wm.m[k] & 0xffffu);
        }
    }
    // two widths per 32-bit scan (16-bit fields; a sub-unit has <= 4096 groups)
    uint32_t A[2], B[2], eA[2], eB[2], tA[2], tB[2];
#pragma unroll
    for (int q = 0; q < 2; q++) {
        const int k0 = 2 * q, k1 = 2 * q + 1;
        A[q] = (uint32_t)(h0[0][k0] + h0[1][k0]) | ((uint32_t)(h0[0][k1] + h0[1][k1]) << 16);
        B[q] = (uint32_t)(cnt[0][k0] - h0[0][k0] + cnt[1][k0] - h0[1][k0]) |
               ((uint32_t)(cnt[0][k1] - h0[0][k1] + cnt[1][k1] - h0[1][k1]) << 16);
        const uint32_t ia = (uint32_t)scan64((int)A[q]), ib = (uint32_t)scan64((int)B[q]);
        tA[q] = (uint32_t)__builtin_amdgcn_readlane((int)ia, 63);
        tB[q] = (uint32_t)__builtin_amdgcn_readlane((int)ib, 63);
        eA[q] = ia - A[q];
        eB[q] = ib - B[q];
    }
    int tot0[4], tot[4], pb[4], np = 0;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const int sh = 16 * (k & 1);
        tot0[k] = (int)((tA[k >> 1] >> sh) & 0xffffu);
        tot[k] = tot0[k] + (int)((tB[k >> 1] >> sh) & 0xffffu);
        pb[k] = np;
        np += (tot[k] + 63) >> 6;
    }
#pragma unroll
    for (int j = 0; j < 2; j++) {
        const int i = 2 * lane + j;
        if (i < nrs) {
            uint32_t *d = info + i * kInfo;
            reinterpret_cast<uint4 *>(d)[0] =
                make_uint4(p0[j], p1[j], ((uint32_t)r[j] << 13) | ((uint32_t)(32 * s[j]) << 20), (uint32_t)ng[j]);
            uint32_t bb = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const int sh = 16 * (k & 1);
                int x0 = (int)((eA[k >> 1] >> sh) & 0xffffu), x1 = (int)((eB[k >> 1] >> sh) & 0xffffu);
                if (j == 1) { // after this lane's first row-slice
                    x0 += h0[0][k];
                    x1 += cnt[0][k] - h0[0][k];
                }
                const uint32_t sb0 = (uint32_t)(64 * pb[k] + x0);
                const uint32_t sb1 = (uint32_t)(64 * pb[k] + tot0[k] + x1 - h0[j][k]);
                d[4 + 3 * k] = m[j][k];
                d[5 + 3 * k] = sb0 | (sb1 << 16);
                d[6 + 3 * k] = rec8[j] + bb;
                bb += (uint32_t)cnt[j][k] << k;
            }
        }
    }
    if (lane == 0) {
        reinterpret_cast<uint4 *>(hdr)[0] = make_uint4((uint32_t)np, (uint32_t)pb[1], (uint32_t)pb[2], (uint32_t)pb[3]);
        reinterpret_cast<uint4 *>(hdr)[1] = make_uint4((uint32_t)tot[0], (uint32_t)tot[1], (uint32_t)tot[2], (uint32_t)tot[3]);
        hdr[8] = 0u; // pass counter
    }
}

template <int kPer> // rounds of kT / 32 row-slices
__device__ __forceinline__ void build_table_n(const Ctx &c, int nrs, int buf)
{
    const int tid = threadIdx.x;
    const uint32_t *info = reinterpret_cast<const uint32_t *>(c.smem + c.L.info) + buf * kMaxRS * kInfo;
    uint32_t *table = reinterpret_cast<uint32_t *>(c.smem + c.L.table);
    const uint32_t g = tid & 31;
    const uint32_t lt = (1u << g) - 1u, hsh = g < 16 ? 0u : 16u, gx = g << 20;
    // all descriptor reads first: two LDS round trips for the whole table
    uint4 d0[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = (tid >> 5) + k * (kT / 32);
        d0[k] = i < nrs ? *reinterpret_cast<const uint4 *>(info + i * kInfo) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t cc[kPer], m[kPer], sb[kPer], cb[kPer];
    bool on[kPer];
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = (tid >> 5) + k * (kT / 32);
        on[k] = g < d0[k].w; // zero for row-slices past the sub-unit
        cc[k] = ((d0[k].x >> g) & 1u) | (((d0[k].y >> g) & 1u) << 1);
        const uint32_t *dc = info + (on[k] ? i : 0) * kInfo + 4 + 3 * cc[k];
        m[k] = dc[0];
        sb[k] = dc[1];
        cb[k] = dc[2];
    }
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        if (on[k]) {
            const uint32_t rank = (uint32_t)__popc(m[k] & lt);
            const uint32_t slot = ((sb[k] >> hsh) & 0xffffu) + rank;
            table[slot] = (cb[k] + (rank << cc[k])) + d0[k].z + gx;
        }
    }
}

// Slot-table entries of rows [ra, rb): thread = (row-slice, group).
// entry = code offset / 8 (13 bits) | row in sub-unit (7 bits) << 13 | group column << 20
__device__ __forceinline__ void build_table(const Ctx &c, int ra, int rb, int buf)
{
    const int nrs = (rb - ra) * c.a.nS;
    constexpr int kRoundRS = kT / 32; // row-slices per round
    static_assert(kMaxRS <= 4 * kRoundRS, "at most four rounds");
    switch ((nrs + kRoundRS - 1) / kRoundRS) {
    case 1: build_table_n<1>(c, nrs, buf); break;
    case 2: build_table_n<2>(c, nrs, buf); break;
    case 3: build_table_n<3>(c, nrs, buf); break;
    default: build_table_n<4>(c, nrs, buf); break;
    }
}

// One pass: 64 slots of width B.
template <int B, int MT>
__device__ __forceinline__ void run_pass(const Ctx &c, int p, int end_slot, const uint32_t *table,
                                         const uint8_t *codes, const uint16_t *scales, const uint32_t *xrec,
                                         float *psum)
{
    constexpr int C = B == 1 ? 0 : B == 2 ? 1 : B == 4 ? 2 : 3;
    const int slot = p * 64 + (int)(threadIdx.x & 63);
    if (slot >= end_slot)
        return;
    const uint32_t e = table[slot];
    const uint32_t code8 = e & 0x1fffu, row = (e >> 13) & 127u, xcol = e >> 20;
    const uint32_t sidx = __umul24(row, (uint32_t)c.a.G) + xcol;
    uint32_t w[2 * B];
    const U2 *src = reinterpret_cast<const U2 *>(codes + code8 * 8u);
#pragma unroll
    for (int k = 0; k < B; k++) {
        const U2 v = src[k];
        w[2 * k] = v.v[0];
        w[2 * k + 1] = v.v[1];
    }
    uint32_t h[32];
    unpack_pairs<B>(w, h);
    const float s = __half2float(__ushort_as_half(scales[sidx]));
#pragma unroll
    for (int m = 0; m < MT; m++) {
        const uint32_t *xr = xrec + ((uint32_t)m * c.a.G + xcol) * kXRec;
        float acc0 = 0.f, acc1 = 0.f; // two chains for instruction-level parallelism
#pragma unroll
        for (int k = 0; k < 8; k += 2) {
            const U4 xa = *reinterpret_cast<const U4 *>(xr + 4 * k);
            const U4 xb = *reinterpret_cast<const U4 *>(xr + 4 * k + 4);
            acc0 = dot2(h[4 * k + 0], xa.v[0], acc0);
            acc1 = dot2(h[4 * k + 4], xb.v[0], acc1);
            acc0 = dot2(h[4 * k + 1], xa.v[1], acc0);
            acc1 = dot2(h[4 * k + 5], xb.v[1], acc1);
            acc0 = dot2(h[4 * k + 2], xa.v[2], acc0);
            acc1 = dot2(h[4 * k + 6], xb.v[2], acc1);
            acc0 = dot2(h[4 * k + 3], xa.v[3], acc0);
            acc1 = dot2(h[4 * k + 7], xb.v[3], acc1);
        }
        const float cc = __uint_as_float(xr[32 + C]);
        psum[m * kPsum + sidx] = s * ((acc0 + acc1) - cc);
    }
}

// x records for all of K: fp16 pairs (x_p, x_{p+32}), then per width
// C_b = sum_p 2^(10-pos_b(p)) (x_p + x_{p+32}) + (2^b-1)/2 sum_j x_j.
// Item = (token, group, part r): pairs 8r..8r+7, from x_{8r..8r+7} and
// x_{32+8r..32+8r+7} (two 16-byte loads where x allows); the 4 items of a
// group are 4 adjacent lanes.  Loading and storing are separate so the loads
// can be issued together with the other prologue loads.
template <int MT>
struct XStage {
    static constexpr int kPer = (MT * 256 * 4 + kT - 1) / kT; // items per thread (G < 256)
    uint4 lo[kPer], hi[kPer];
};

template <int MT>
__device__ __forceinline__ void stage_x_load(const Ctx &c, XStage<MT> &xs)
{
    const int tid = threadIdx.x;
    const int G = c.a.G;
    const int items = MT * G * 4;
    const bool vec = (c.a.ldx % 4) == 0 && ((uintptr_t)c.a.x % 8) == 0; // dword-aligned 16-byte loads
#pragma unroll
    for (int k = 0; k < XStage<MT>::kPer; k++) {
        const int i = tid + k * kT;
        xs.lo[k] = xs.hi[k] = make_uint4(0u, 0u, 0u, 0u);
        if (i < items) {
            const int r = i & 3, g = (i >> 2) % G, m = (i >> 2) / G;
            const uint16_t *p = c.a.x + (uint64_t)m * c.a.ldx + 64ull * g + 8 * r;
            if (vec) {
                xs.lo[k] = *reinterpret_cast<const uint4 *>(p);
                xs.hi[k] = *reinterpret_cast<const uint4 *>(p + 32);
            } else {
                xs.lo[k] = make_uint4(p[0] | ((uint32_t)p[1] << 16), p[2] | ((uint32_t)p[3] << 16),
                                      p[4] | ((uint32_t)p[5] << 16), p[6] | ((uint32_t)p[7] << 16));
                xs.hi[k] = make_uint4(p[32] | ((uint32_t)p[33] << 16), p[34] | ((uint32_t)p[35] << 16),
                                      p[36] | ((uint32_t)p[37] << 16), p[38] | ((uint32_t)p[39] << 16));
            }
        }
    }
}

// Sum over each aligned group of 4 lanes, in a fixed order (DPP quad moves).
__device__ __forceinline__ float quad_sum(float v)
{
    v += dpp_f<0xB1>(v); // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v); // quad_perm [2, 3, 0, 1]
    return v;
}

template <int MT>
__device__ __forceinline__ void stage_x_store(const Ctx &c, const XStage<MT> &xs, uint32_t *xrec)
{
    const int tid = threadIdx.x;
    const int G = c.a.G;
    const int items = MT * G * 4;
#pragma unroll
    for (int k = 0; k < XStage<MT>::kPer; k++) {
        const int i = tid + k * kT;
        if (i >= items) // whole groups of 4 lanes drop out together
            break;
        const int r = i & 3, g = (i >> 2) % G, m = (i >> 2) / G;
        const uint32_t lo[4] = {xs.lo[k].x, xs.lo[k].y, xs.lo[k].z, xs.lo[k].w};
        const uint32_t hi[4] = {xs.hi[k].x, xs.hi[k].y, xs.hi[k].z, xs.hi[k].w};
        uint32_t pr[8];
#pragma unroll
        for (int h = 0; h < 4; h++) {
            pr[2 * h] = __builtin_amdgcn_perm(hi[h], lo[h], 0x05040100u);     // (x_p, x_{p+32})
            pr[2 * h + 1] = __builtin_amdgcn_perm(hi[h], lo[h], 0x07060302u); // next p
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
            // the mantissa position of pair t depends on its index inside its word
            c1 = fmaf((float)(1 << (10 - pair_pos<1>(t & 15))), sp, c1);
            c2 = fmaf((float)(1 << (10 - pair_pos<2>(t & 7))), sp, c2);
            c4 = fmaf((float)(1 << (10 - pair_pos<4>(t & 3))), sp, c4);
        }
        // fixed-order tree over the 4 parts (DPP lane moves, no LDS)
        X = quad_sum(X);
        c1 = quad_sum(c1);
        c2 = quad_sum(c2);
        c4 = quad_sum(c4);
        if (r == 0)
            *reinterpret_cast<U4 *>(xr + 32) = U4{{__float_as_uint(fmaf(0.5f, X, c1)),
                                                    __float_as_uint(fmaf(1.5f, X, c2)),
                                                    __float_as_uint(fmaf(7.5f, X, c4)),
                                                    __float_as_uint(fmaf(127.5f, X, 1024.f * X))}};
    }
}

template <int MT>
__global__ __launch_bounds__(kT) void k_gemv_stream(SArgs args)
{
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // this workgroup's matrix: the last one whose first workgroup is <= blockIdx.x
    SArgs a = args;
    int wg0 = 0;
#pragma unroll
    for (int i = 0; i < kMaxMats; i++) {
        if (i < args.nmat && (int)blockIdx.x >= args.mats[i].wg0) {
            a.blob = args.mats[i].blob;
            a.off_row_off = args.mats[i].off_row_off;
            a.off_slice_off = args.mats[i].off_slice_off;
            a.off_wmap = args.mats[i].off_wmap;
            a.off_scales = args.mats[i].off_scales;
            a.off_codes = args.mats[i].off_codes;
            a.y = args.mats[i].y;
            a.N = args.mats[i].N;
            a.ldy = args.mats[i].ldy;
            wg0 = args.mats[i].wg0;
        }
    }
    Ctx c;
    c.a = a;
    c.n0 = ((int)blockIdx.x - wg0) * a.rows;
    if (c.n0 >= a.N)
        return;
    c.R = min(a.rows, a.N - c.n0);
    c.smem = smem;
    c.L = s_layout(MT, a.G, a.rows, a.nS, a.cap);
    const int nS = a.nS, G = a.G, R = c.R;
    uint32_t *rowoff = reinterpret_cast<uint32_t *>(smem + c.L.rowoff);
    uint32_t *sloff = reinterpret_cast<uint32_t *>(smem + c.L.sloff);
    uint32_t *wmap = reinterpret_cast<uint32_t *>(smem + c.L.wmap);
    uint32_t *xrec = reinterpret_cast<uint32_t *>(smem + c.L.x);
    const uint32_t *table = reinterpret_cast<const uint32_t *>(smem + c.L.table);
    float *psum = reinterpret_cast<float *>(smem + c.L.psum);
    float *ybuf = reinterpret_cast<float *>(smem + c.L.ybuf);

    // ---- metadata of this workgroup's rows, the activations, and (in every
    // wave) the row offsets of the first kMaxRS rows: the first sub-unit's copy
    // is issued and described as soon as they arrive, before x is staged
    int ra = 0, rb, rc;
    {
        const uint32_t *g_row = reinterpret_cast<const uint32_t *>(a.blob + a.off_row_off) + c.n0;
        const uint32_t *g_slo = reinterpret_cast<const uint32_t *>(a.blob + a.off_slice_off) + (uint64_t)c.n0 * nS;
        const uint32_t *g_wm = reinterpret_cast<const uint32_t *>(a.blob + a.off_wmap) + 2ull * c.n0 * nS;
        const int nrs = R * nS;
        uint32_t win[kMaxRS / 64];
#pragma unroll
        for (int h = 0; h < kMaxRS / 64; h++)
            win[h] = g_row[min(lane + 1 + 64 * h, R)];
        const uint32_t win0 = g_row[0];
        XStage<MT> xs;
        stage_x_load<MT>(c, xs);
        // wave 0 also reads the first sub-unit's row-slice inputs into registers
        // (up to kMaxRS row-slices; build_info masks those past the sub-unit)
        InfoIn in0;
        if (wave == 0) {
#pragma unroll
            for (int j = 0; j < 2; j++) {
                const int i = 2 * lane + j;
                const bool live = i < nrs;
                const int r = (int)(((uint32_t)i * (uint32_t)a.inv_nS) >> 16);
                in0.p0[j] = live ? g_wm[2 * i] : 0u;
                in0.p1[j] = live ? g_wm[2 * i + 1] : 0u;
                in0.slo[j] = live ? g_slo[i] : 0u;
                in0.roff[j] = live ? g_row[r] : 0u; // made relative after the loads land
            }
        }
        uint32_t r0 = 0, r1 = 0, sl = 0, w0 = 0, w1 = 0;
        if (tid <= R)
            r0 = g_row[tid];
        if (tid + kT <= R)
            r1 = g_row[tid + kT];
        if (tid < nrs)
            sl = g_slo[tid];
        if (tid < 2 * nrs)
            w0 = g_wm[tid];
        if (tid + kT < 2 * nrs)
            w1 = g_wm[tid + kT];
        {
            // rows of the first sub-unit, from registers (same rule as next_end).
            // When the whole block fits both ring slots it is one sub-unit.
            const int kmax = min(kMaxRS / nS, R);
            uint32_t endR = 0;
#pragma unroll
            for (int h = 0; h < kMaxRS / 64; h++)
                if ((R - 1) >> 6 == h)
                    endR = __shfl(win[h], (R - 1) & 63);
            const bool single = R <= kmax && (endR - win0) * 128u <= 2u * (uint32_t)a.cap;
            const uint32_t cap = single ? 2u * (uint32_t)a.cap : (uint32_t)a.cap;
            int n = 0;
#pragma unroll
            for (int h = 0; h < kMaxRS / 64; h++) {
                const int k = lane + 1 + 64 * h;
                n += (int)__popcll(__ballot(k <= kmax && (win[h] - win0) * 128u <= cap));
            }
            rb = n;
            // the row offset that ends it: lane (rb - 1) % 64 of window half (rb - 1) / 64
            const int src = (rb - 1) & 63;
            uint32_t end = __shfl(win[0], src);
#pragma unroll
            for (int h = 1; h < kMaxRS / 64; h++)
                if ((rb - 1) >> 6 == h)
                    end = __shfl(win[h], src);
            Copy k0 = make_copy(c, win0, end, 0, rb, 0, 0);
            issue_all(c, k0);
            if (wave == 0) {
                in0.roff[0] -= win0;
                in0.roff[1] -= win0;
                to_slice_major(in0, rb, nS);
                build_info(c, 0, rb, 0, in0);
            }
        }
        // no global loads after this point of the prologue: the compiler's waits
        // for the loads above cannot pick up the copy just issued
        stage_x_store<MT>(c, xs, xrec);
        if (tid <= R)
            rowoff[tid] = r0;
        if (tid + kT <= R)
            rowoff[tid + kT] = r1;
        if (tid < nrs)
            sloff[tid] = sl;
        if (tid < 2 * nrs)
            wmap[tid] = w0;
        if (tid + kT < 2 * nrs)
            wmap[tid + kT] = w1;
    }
    __syncthreads();

    // ---- sub-units u and u+1 start at rows ra and rb; rc ends u+1
    rc = next_end(c, rb);
    int slot = 0;

    for (int u = 0; ra < R; u++) {
        const int buf = u & 1;
        build_table(c, ra, rb, buf);
        wait_vm(0); // this wave's chunks of u (the only vector-memory ops in the loop)
        __syncthreads();

        // ---- passes of u, handed out through an LDS counter; wave 0 first
        // describes u+1.  The copy of u+1 into the slot that u-1 used goes out
        // one chunk per pass.
        int l1 = 0;
        {
            const uint32_t *rowoff_l = rowoff;
            Copy k1 = make_copy(c, rowoff_l[rb], rowoff_l[rc], rb, rc, slot ^ 1, u + 1);
            if (rb >= R)
                k1.n = 0;
            if (wave == 0 && rb < R) {
                InfoIn in;
                info_in_lds(c, rb, rc, in);
                build_info(c, rb, rc, buf ^ 1, in);
            }
            uint32_t *hdr = reinterpret_cast<uint32_t *>(smem + c.L.hdr) + buf * 16;
            const uint4 h0 = *reinterpret_cast<const uint4 *>(hdr);
            const uint4 h1 = *reinterpret_cast<const uint4 *>(hdr + 4);
            const int np = (int)h0.x, pb1 = (int)h0.y, pb2 = (int)h0.z, pb3 = (int)h0.w;
            const uint8_t *codes = smem + slot_codes(c, slot);
            const uint64_t s0 = (uint64_t)(c.n0 + ra) * G * 2u;
            const uint16_t *scales = reinterpret_cast<const uint16_t *>(smem + slot_scales(c, slot) + (s0 & 15u));
            for (;;) {
                int p = 0;
                if (lane == 0)
                    p = (int)atomicAdd(hdr + 8, 1u);
                l1 += issue_next(c, k1);
                p = __builtin_amdgcn_readfirstlane(p);
                if (p >= np)
                    break;
                if (p < pb1)
                    run_pass<1, MT>(c, p, (int)h1.x, table, codes, scales, xrec, psum);
                else if (p < pb2)
                    run_pass<2, MT>(c, p, 64 * pb1 + (int)h1.y, table, codes, scales, xrec, psum);
                else if (p < pb3)
                    run_pass<4, MT>(c, p, 64 * pb2 + (int)h1.z, table, codes, scales, xrec, psum);
                else
                    run_pass<8, MT>(c, p, 64 * pb3 + (int)h1.w, table, codes, scales, xrec, psum);
            }
            l1 += issue_all(c, k1);
        }
        __syncthreads();

        // ---- rows of u: 8 lanes per row, fixed summation order
        {
            const int nr = rb - ra;
            const int j = tid >> 3, q = tid & 7;
            if (j < nr) {
#pragma unroll
                for (int m = 0; m < MT; m++) {
                    const float *ps = psum + m * kPsum + j * G;
                    float v = 0.f;
                    for (int k = q; k < G; k += 8)
                        v += ps[k];
                    v = group_sum<8>(v);
                    if (q == 0)
                        ybuf[m * a.rows + ra + j] = v;
                }
            }
        }
        // ---- advance
        (void)l1;
        ra = rb;
        rb = rc;
        rc = next_end(c, rc);
        slot ^= 1;
    }
    // ---- y of this workgroup's rows, coalesced
    __syncthreads();
    for (int i = tid; i < MT * R; i += kT) {
        const int m = i / R, r = i - m * R;
        const float v = ybuf[m * a.rows + r];
        const uint64_t o = (uint64_t)m * a.ldy + c.n0 + r;
        if (a.yt == VBQ_F16)
            reinterpret_cast<__half *>(a.y)[o] = __float2half_rn(v);
        else
            reinterpret_cast<float *>(a.y)[o] = v;
    }
}

template <int MT>
vbq_status launch_stream(const SArgs &a, int grid, size_t smem, hipStream_t stream)
{
    VBQ_TRY(dynamic_lds_once((const void *)k_gemv_stream<MT>, 160 * 1024));
    hipLaunchKernelGGL(k_gemv_stream<MT>, dim3(grid), dim3(kT), smem, stream, a);
    return launch_status();
}

// Launch plan for n matrices of the same K sharing x, one workgroup per CU:
// rows per workgroup, grid, sub-unit cap and LDS bytes.  False when the
// streaming kernel does not apply.
struct Plan {
    int rows, grid, cap;
    uint32_t smem;
};

bool make_plan(const StreamItem *items, int n, int M, Plan &p)
{
    const int G = (int)items[0].L->G, nS = (int)items[0].L->nS;
    if (nS > kMaxRS)
        return false;
    int64_t total = 0;
    for (int i = 0; i < n; i++)
        total += items[i].L->N;
    const int wgs = current_device_cus();
    int rows = (int)((total + wgs - 1) / wgs);
    rows = std::max(1, std::min(rows, kMetaRS / nS));
    const uint32_t budget = 160u * 1024u;
    // the largest sub-unit (1 KiB steps) that fits; every row record (8 bytes
    // per bit of width, padded to 128) must fit one sub-unit
    p.cap = 0;
    for (int cand = kMaxCap; cand >= 8192; cand -= 1024) {
        if ((uint64_t)G * 64u + 128u > (uint64_t)cand)
            break;
        if (s_layout(M, G, rows, nS, cand).total <= budget) {
            p.cap = cand;
            break;
        }
    }
    if (!p.cap)
        return false;
    p.rows = rows;
    p.smem = s_layout(M, G, rows, nS, p.cap).total;
    p.grid = 0;
    for (int i = 0; i < n; i++)
        p.grid += ((int)items[i].L->N + rows - 1) / rows;
    return true;
}

template <int MT>
vbq_status run(const StreamItem *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt, const Plan &p,
               hipStream_t stream)
{
    const int G = (int)items[0].L->G, nS = (int)items[0].L->nS;
    SArgs a = {};
    a.G = G;
    a.nS = nS;
    a.M = M;
    a.x = x;
    a.ldx = ldx;
    a.yt = (int)yt;
    a.rows = p.rows;
    a.cap = p.cap;
    a.inv_nS = (65536 + nS - 1) / nS;
    a.nmat = n;
    int wg = 0;
    for (int i = 0; i < n; i++) {
        const vbq_layout *L = items[i].L;
        SMat &m = a.mats[i];
        m.blob = (const uint8_t *)items[i].blob;
        m.off_row_off = L->off_row_off;
        m.off_slice_off = L->off_slice_off;
        m.off_wmap = L->off_wmap;
        m.off_scales = L->off_scales;
        m.off_codes = L->off_codes;
        m.y = items[i].y;
        m.N = (int)L->N;
        m.ldy = items[i].ldy;
        m.wg0 = wg;
        wg += (m.N + p.rows - 1) / p.rows;
    }
    return launch_stream<MT>(a, p.grid, p.smem, stream);
}

} // namespace

namespace vbq {

bool stream_gemv_shared(const StreamItem *items, int n, int M, const uint16_t *x, int ldx, vbq_dtype yt,
                        hipStream_t stream, vbq_status *st)
{
    if (M < 1 || M > 2 || n < 1 || n > kMaxMats)
        return false;
    for (int i = 1; i < n; i++)
        if (items[i].L->K != items[0].L->K)
            return false;
    Plan p;
    if (!make_plan(items, n, M, p))
        return false;
    *st = M == 1 ? run<1>(items, n, M, x, ldx, yt, p, stream) : run<2>(items, n, M, x, ldx, yt, p, stream);
    return true;
}

bool stream_applies(const vbq_layout *L, int M)
{
    if (M < 1 || M > 2)
        return false;
    const StreamItem it{L, nullptr, nullptr, 0};
    Plan p;
    return make_plan(&it, 1, M, p);
}

bool stream_gemv(const GemvCall &g, vbq_status *st)
{
    const StreamItem it{g.L, g.blob, g.y, g.ldy};
    return stream_gemv_shared(&it, 1, g.M, g.x, g.ldx, g.yt, g.stream, st);
}

} // namespace vbq
