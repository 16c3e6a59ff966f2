// q8_matmul.hip -- the narrow-batch q8_0 matmul for gfx950.
//
// "Batched decode: co-decode N live sessions in one GPU pass" (antirez/ds4 PR
// #530), section "Why it's worth it -- the narrow-batch matmul": decode is
// memory-bound, so each 32-weight block is read from memory once and dotted
// against the activation blocks of every live token.  Here:
//
//   S[t,n,b] = sum_i qw[n,32b+i] * qx[slot_t,32b+i]          exact int32
//   y[t,n]  += float(S) * (float(dw[n,b]) * float(dx[slot_t,b]))
//
// with one fused multiply-add per term; dw*dx is exact in fp32 (two 11-bit
// significands).  The fp32 summation follows one tree per (N, K), whatever
// the live batch or execution strategy:
//   * K is cut into S splits (contiguous runs of 256-value super-chunks),
//     each split into KW wave slices;
//   * a wave adds its terms in ascending block order;
//   * level 1: a split's partial is the sum of its KW wave partials in order;
//   * level 2: the output is the sum of the S split partials in order.
// The plain entry point evaluates the whole tree in one workgroup of S*KW
// waves (levels 1 and 2 through LDS).  The workspace entry point runs the S
// splits of a row block as S workgroups: each evaluates level 1 and writes
// its partial to the workspace; the last of them to arrive (a counter per
// row block) evaluates level 2, writes Y and rearms the counter.  Both give
// the same bits, and
// so does the DOT4 engine below, so a token's output never depends on
// n_live, on the other tokens or on the entry point.
//
// Two int8 dot engines compute S, with the same accumulation order, so their
// results are bit-identical:
//   * MFMA: one v_mfma_i32_16x16x32_i8 per (16 rows, block) dots the block
//     against all 16 activation slots at once.  A = weights (row = lane & 15),
//     B = slots (slot = lane & 15), D[row][slot] -> lane holds slot lane & 15
//     for rows 4*(lane >> 4) + r, so a lane needs one slot's activation
//     scales and four consecutive rows' weight scales.  Both come once per
//     super-chunk, one dword per lane, and reach the lanes that need them
//     through DPP row broadcasts and permlane swaps.  The cost is the same
//     for any n_live: the weight stream is what the kernel spends its time
//     on.  Tokens take their slot's column when the outputs are stored.  A
//     wave covers RG row groups, so each activation load feeds 16*RG rows.
//   * DOT4: one output row per lane, v_dot4 over the row's 32 bytes against
//     the token's block (wave-uniform, so it comes through scalar loads).  Its
//     VALU work grows with n_live.
//
// Token slots come from batch_index ("[feature] Enable Dynamic Batching",
// section "Objective": batch_index selects rows of a fixed, fully sized
// buffer).  The slot buffer has the packed layout of a 16-row matrix, so the
// activation operand of one chunk for all 16 slots is 1 KB contiguous.  A
// slot index outside [0,16) is never read through (slot 0 is read instead)
// and its output row is written as NaN.

#include "q8_internal.h"

#include <math.h>

#include <algorithm>
#include <type_traits>
#ifdef Q8_TIMELINE
#include <mutex>
#endif

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxKs = 16;             // waves per workgroup at most
constexpr size_t kMaxLds = 64 * 1024;  // dynamic LDS per workgroup we allow

__device__ inline uint4 ld16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// 16-byte load marked non-temporal (streamed once, not worth caching).
__device__ inline uint4 ld16_nt(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The activation slot buffer is never written while a matmul runs, so a
// wave-uniform address into it may be read through the scalar cache.
typedef __attribute__((address_space(4))) const u32x4 cu32x4;

__device__ inline _Float16 half_bits(uint32_t w, int hi) {
    return __builtin_bit_cast(_Float16, (uint16_t)(w >> (16 * hi)));
}

__device__ inline int live_slot(const int32_t* __restrict__ bidx, int n_live, int t) {
    const int s = bidx[t < n_live ? t : 0];
    return (s >= 0 && s < kMaxSlots) ? s : 0;
}

__device__ inline bool slot_bad(const int32_t* __restrict__ bidx, int t) {
    const int s = bidx[t];
    return s < 0 || s >= kMaxSlots;
}

// One term of the sum: acc + S * (dw * dx), the product of the two binary16
// scales being exact in fp32.
__device__ inline float term_fma(int S, _Float16 dw, _Float16 dx, float acc) {
    const float p = __builtin_fmaf((float)dw, (float)dx, 0.0f);
    return __builtin_fmaf((float)S, p, acc);
}

struct MmArgs {
    const uint8_t* wq;    // weights: packed q region
    const uint16_t* wd;   // weights: packed scale region
    const uint8_t* xq;    // activation slots: q region (16-row packed layout)
    const uint16_t* xd;   // activation slots: scale region
    const int32_t* bidx;  // batch_index
    float* Y;
    uint8_t* recs;        // workspace: one record per row block (see split_record)
    int64_t N;
    int64_t G;
    int KB, NSC, n_live;
    int S, KW;            // summation tree: splits, wave slices per split
    int n_rb;             // row blocks (RG row groups each)
    int n_whole;          // leading row blocks whose workgroup is one wave that evaluates
                          // every split in turn (KW == 1); SPLIT: the rest run as S
                          // split workgroups each
    int CT;               // slot column tiles (16 slots each)
    int y_vec4;           // N % 4 == 0 and Y 16-byte aligned: rows stored as float4
    int64_t xq_gs;        // slot buffer: bytes per 16 slots of the q region
    int64_t xd_gs;        // slot buffer: halves per 16 slots of the scale region
    // fused pre-quantisation (FUSED kernels only)
    const float* X;       // fp32 activations [n_rows][K]
    int n_rows;
    int P;                // producer workgroups, blockIdx.x < P
    int n_cons;           // consumer (matmul) workgroups
    int max_spins;        // polls of the bounded wait
    uint32_t* qflag;      // producer groups that have published their slots
    uint32_t* qexit;      // workgroups (producers and consumers) that are done
    uint32_t* qflag_sub;  // kSubCounters producer counters, kSubStride apart
    uint32_t* qexit_sub;  // kSubCounters exit counters, kSubStride apart
    uint32_t* qready;     // kReadyCopies "slots published" flags, kReadyStride apart
    uint32_t* timeouts;   // matmul workgroups whose wait ran out (never cleared here)
#ifdef Q8_TIMELINE
    uint64_t* tl;         // wave timeline records (null: none), kStampWords per wave
    int64_t tl_waves;     // records the buffer holds
#endif
};

// Per-wave timeline.  In the timeline build (Q8_TIMELINE) every wave of a
// matmul launch reads the 100 MHz real-time counter at fixed points and lane
// 0 writes them, with the wave's XCC and hardware ids, to a record of
// kStampWords uint64 (wave index blockIdx.x * waves + wave); see
// include/q8timeline.h for the fields.  In the product build every call
// below is empty and the kernel is unchanged.
constexpr int kStampWords = 8;

struct WaveStamps {
#ifdef Q8_TIMELINE
    uint64_t t[kStampWords];
    __device__ WaveStamps() {
#pragma unroll
        for (int i = 0; i < kStampWords; ++i) t[i] = 0;
        t[0] = __builtin_amdgcn_s_memrealtime();
        uint32_t hw, xcc;
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
        asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
        t[7] = ((uint64_t)(xcc & 0xF) << 32) | hw;
    }
    __device__ void mark(int i) { t[i] = __builtin_amdgcn_s_memrealtime(); }
    __device__ void mark_once(int i) {
        if (t[i] == 0) mark(i);
    }
    // stores complete first, so that the next mark times them
    __device__ void drain() { __builtin_amdgcn_s_waitcnt(0); }
    __device__ void write(const MmArgs& a, int64_t wave, int lane) const {
        if (a.tl == nullptr || lane != 0 || wave >= a.tl_waves) return;
#pragma unroll
        for (int i = 0; i < kStampWords; ++i) a.tl[wave * kStampWords + i] = t[i];
    }
#else
    __device__ void mark(int) {}
    __device__ void mark_once(int) {}
    __device__ void drain() {}
    __device__ void write(const MmArgs&, int64_t, int) const {}
#endif
};

// Super-chunk range [lo, hi) of wave slice k of split s (NSC <= 2^16, so 32-bit
// products are exact).
__device__ inline void slice_range(int NSC, int S, int KW, int s, int k, int& lo, int& hi) {
    const int s0 = s * NSC / S, s1 = (s + 1) * NSC / S;
    const int len = s1 - s0;
    lo = s0 + k * len / KW;
    hi = s0 + (k + 1) * len / KW;
}

// Level 1 of the tree for element e of a tile of E elements: the partial of
// split s from the KW wave partials red[(s*KW + k)*E + e], k ascending.
__device__ inline float split_sum(const float* red, int E, int e, int s, int KW) {
    float p = red[(s * KW) * E + e];
    for (int k = 1; k < KW; ++k) p += red[(s * KW + k) * E + e];
    return p;
}

// Levels 1 and 2 when all S*KW wave partials are in this workgroup's LDS.
__device__ inline float tree_sum(const float* red, int E, int e, int S, int KW) {
    float y = split_sum(red, E, e, 0, KW);
    for (int s = 1; s < S; ++s) y += split_sum(red, E, e, s, KW);
    return y;
}

// The workspace of a split execution is one record per row block that runs
// as split workgroups: the block's arrival counter alone in a 256-byte
// line, then room for kRecordSplits split partials of its E-element tile.
// Every split shape runs at most kRecordSplits splits of a one-row-group,
// one-column-tile tile (E = 256), so the records of every shape have the
// same stride: a counter of one shape always sits where every other shape
// keeps a counter, never where partials were.  A workspace whose counters
// every call rearms may therefore serve matrices of any shape in turn.
constexpr int64_t kRecordHead = 256;
constexpr int kRecordSplits = 4;

__host__ __device__ inline int64_t record_bytes(int S, int E) {
    return kRecordHead + (int64_t)(S > kRecordSplits ? S : kRecordSplits) * E *
                             (int64_t)sizeof(float);
}

__device__ inline uint32_t* record_counter(uint8_t* recs, int rb, int S, int E) {
    return reinterpret_cast<uint32_t*>(recs + rb * record_bytes(S, E));
}

__device__ inline float* record_part(uint8_t* recs, int rb, int S, int E, int split) {
    return reinterpret_cast<float*>(recs + rb * record_bytes(S, E) + kRecordHead) + split * E;
}

// ------------------------------------------------------------------------
// MFMA engine
// ------------------------------------------------------------------------

// The MFMA engine dots every chunk against all 16 activation slots, whatever
// the live batch: one 16x16x32 MFMA costs the same for 1 or 16 columns, and
// nothing in the streaming loop then depends on batch_index.  The tokens are
// picked out of the slot columns only when the outputs are stored (token t
// takes slot batch_index[t]'s column), which gives each token exactly the
// arithmetic of its own slot.  A slot no token names is computed and
// dropped; its values, whatever they are, never reach another column.
//
// Each wave streams its K-slice one chunk (2 blocks, 1 KB per row group) at a
// time through a ring of D chunks: it dots the oldest chunk and issues the
// loads of the chunk D places ahead, so every wave keeps a steady stream of
// requests in flight.  A slice is a whole number of super-chunks (4 chunks),
// so with D dividing 4 the ring needs no bounds tests: every load and every
// wait is the same in every turn of the loop.

typedef long v2i64 __attribute__((ext_vector_type(2)));

__device__ inline v2i64 ld16_v2(const void* p) {
    return *reinterpret_cast<const v2i64*>(p);
}

__device__ inline v2i64 ld16_v2_nt(const void* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v2i64*>(p));
}

// Operands of one chunk for RG row groups and CT column tiles of 16 slots.
// The scales are not part of it: they come once per super-chunk (see
// load_scales).
template <int RG, int CT>
struct Chunk {
    v2i64 w[RG];       // weights: this lane's A operands of blocks 2c, 2c+1
    v2i64 aq[CT];      // slot 16*ct + (lane & 15): B operands of blocks 2c, 2c+1
};

// Chunk cg (global chunk index along K) for RG row groups: the weights (1 KB
// contiguous for the wave per row group).
template <int RG, int CT, bool NTW>
__device__ inline void load_chunk_w(Chunk<RG, CT>& ch, int cg, const uint8_t* wrow,
                                    int64_t g_stride_q) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const uint8_t* p = wrow + rg * g_stride_q + (int64_t)cg * kChunkBytes;
        ch.w[rg] = NTW ? ld16_v2_nt(p) : ld16_v2(p);
    }
}

// Weight scales of super-chunk sc for RG row groups: its 4 chunks x 16 rows
// x 2 blocks are 64 dwords, 256 contiguous bytes, and each lane loads one of
// them, so the wave reads every scale once.  Lane (tq, j) = (lane >> 4,
// lane & 15) takes row 4*tq + (j & 3) of chunk j >> 2; the lanes of row tq of
// the wave between them hold everything lanes tq*16 .. tq*16+15 need (rows
// 4*tq .. 4*tq+3), and chunk_scale hands each its value with a row broadcast.
// wsrow already points at this lane's dword in super-chunk 0.
template <int RG>
__device__ inline void load_scales(uint32_t ws[RG], int sc, const uint16_t* wsrow,
                                   int64_t g_stride_d) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
        ws[rg] = *reinterpret_cast<const uint32_t*>(wsrow + rg * g_stride_d +
                                                    (int64_t)sc * (4 * kChunkDBytes / 2));
}

// Row 4*tq + r, chunk C of the super-chunk: the dword of lane tq*16 + 4*C + r
// (DPP row_newbcast: every lane of a 16-lane row reads lane 4*C + r of it).
template <int C, int R>
__device__ inline uint32_t chunk_scale(uint32_t ws) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)ws, 0x150 + 4 * C + R, 0xf, 0xf, true);
}

template <int RG, int CT>
__device__ inline void load_chunk_a(Chunk<RG, CT>& ch, int cg, const uint8_t* xa, int64_t xq_gs) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) ch.aq[ct] = ld16_v2(xa + ct * xq_gs + (int64_t)cg * kChunkBytes);
}

template <int RG, int CT, bool NTW>
__device__ inline void load_chunk(Chunk<RG, CT>& ch, int cg, const uint8_t* wrow,
                                  int64_t g_stride_q, const uint8_t* xa, int64_t xq_gs) {
    load_chunk_w<RG, CT, NTW>(ch, cg, wrow, g_stride_q);
    load_chunk_a<RG, CT>(ch, cg, xa, xq_gs);
}

// Slot scales of super-chunk sc for CT column tiles: 4 chunks x 16 slots x 2
// blocks, 64 dwords, one per lane: lane l takes chunk l >> 4 of slot l & 15,
// which is the dword l of the super-chunk.  xsrow points at this lane's dword
// in super-chunk 0 of tile 0.
template <int CT>
__device__ inline void load_slot_scales(uint32_t xs[CT], int sc, const uint16_t* xsrow,
                                        int64_t xd_gs) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        xs[ct] = *reinterpret_cast<const uint32_t*>(xsrow + ct * xd_gs +
                                                    (int64_t)sc * (4 * kChunkDBytes / 2));
}

// The same loads as buffer loads, for the multi-tile kernels.  A lane's
// address is then a buffer descriptor's base (scalar registers) + a
// wave-uniform offset (a scalar register) + this lane's byte offset (a
// vector register set once), so an address costs scalar adds only.  Through
// one per-lane 64-bit pointer each load costs a 64-bit vector add: 30 per
// super-chunk at four column tiles, where the VALU is the bottleneck.  The
// one-tile kernels wait on memory, not on the VALU; they keep the global
// form, for which their ring depths were measured.  Offsets stay below 2^31:
// a row block's weights are under 1 GiB (K < 2^24, at most 4 row groups),
// the slot tiles under 2^30 bytes.
struct Src {
    __amdgpu_buffer_rsrc_t rsrc;
    uint32_t lane;  // this lane's byte offset
};

// Operand of the streaming loop: `n` elements from base, this lane's at
// element lane_el: a per-lane pointer (global form) or a descriptor (BUF).
// The descriptor: stride 0 (a raw byte range), loads at or past the end
// read zero, word 3 the gfx9 32-bit data format.
template <bool BUF, typename T>
__device__ inline auto operand(const T* base, int64_t n, int lane_el) {
    if constexpr (BUF) {
        const int64_t bytes = min(n * (int64_t)sizeof(T), (int64_t)0xffffffffu);
        return Src{__builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), (short)0,
                                                     (int)(uint32_t)bytes, 0x00020000),
                   (uint32_t)(lane_el * (int)sizeof(T))};
    } else {
        return base + lane_el;
    }
}

// aux 2: the non-temporal hint (streamed once, not worth caching)
template <bool NT>
__device__ inline v2i64 ld16_v2(const Src& s, int off) {
    return __builtin_bit_cast(
        v2i64, __builtin_amdgcn_raw_buffer_load_b128(s.rsrc, (int)s.lane, off, NT ? 2 : 0));
}

__device__ inline uint32_t ld4(const Src& s, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(s.rsrc, (int)s.lane, off, 0);
}

// The helpers above for a buffer operand; strides in the same units (bytes
// for weights and slots, halves for scales), offsets in 32 bits (64-bit
// ones cost scalar register pairs, and the four-tile kernels then run out of
// registers).
template <int RG, int CT, bool NTW>
__device__ inline void load_chunk_w(Chunk<RG, CT>& ch, int cg, const Src& wq,
                                    int64_t g_stride_q) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
        ch.w[rg] = ld16_v2<NTW>(wq, rg * (int)g_stride_q + cg * kChunkBytes);
}

template <int RG>
__device__ inline void load_scales(uint32_t ws[RG], int sc, const Src& wd, int64_t g_stride_d) {
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
        ws[rg] = ld4(wd, 2 * (rg * (int)g_stride_d + sc * (4 * kChunkDBytes / 2)));
}

template <int RG, int CT>
__device__ inline void load_chunk_a(Chunk<RG, CT>& ch, int cg, const Src& xq, int64_t xq_gs) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        ch.aq[ct] = ld16_v2<false>(xq, ct * (int)xq_gs + cg * kChunkBytes);
}

template <int RG, int CT, bool NTW>
__device__ inline void load_chunk(Chunk<RG, CT>& ch, int cg, const Src& wq, int64_t g_stride_q,
                                  const Src& xq, int64_t xq_gs) {
    load_chunk_w<RG, CT, NTW>(ch, cg, wq, g_stride_q);
    load_chunk_a<RG, CT>(ch, cg, xq, xq_gs);
}

template <int CT>
__device__ inline void load_slot_scales(uint32_t xs[CT], int sc, const Src& xd, int64_t xd_gs) {
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
        xs[ct] = ld4(xd, 2 * (ct * (int)xd_gs + sc * (4 * kChunkDBytes / 2)));
}

// Lane l needs chunk c's dword of its slot l & 15, which lane 16*c + (l & 15)
// holds: row c of the wave copied to all four 16-lane rows.  A 32-lane swap
// of the wave with itself gives rows 0101 and 2323, a 16-lane swap of either
// with itself then rows 0000 and 1111 (2222 and 3333).  One column tile
// keeps all four copies for the super-chunk; wider tiles, short of
// registers, make each chunk's copy when it is used.
template <int CT>
struct SlotScales {
    uint32_t xb[CT][CT == 1 ? 4 : 1];

    __device__ inline void prepare(const uint32_t xs[CT]) {
        if constexpr (CT == 1) {
            const auto p = __builtin_amdgcn_permlane32_swap(xs[0], xs[0], false, false);
            const auto q = __builtin_amdgcn_permlane16_swap(p[0], p[0], false, false);
            const auto r = __builtin_amdgcn_permlane16_swap(p[1], p[1], false, false);
            xb[0][0] = q[0];
            xb[0][1] = q[1];
            xb[0][2] = r[0];
            xb[0][3] = r[1];
        } else {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) xb[ct][0] = xs[ct];
        }
    }

    template <int C>
    __device__ inline uint32_t get(int ct) const {
        if constexpr (CT == 1) {
            return xb[0][C];
        } else {
            const auto p = __builtin_amdgcn_permlane32_swap(xb[ct][0], xb[ct][0], false, false);
            const uint32_t h = p[C >> 1];
            return __builtin_amdgcn_permlane16_swap(h, h, false, false)[C & 1];
        }
    }
};

// f(integral_constant<int, J>) for J = 0 .. N-1, in order.
template <int J, int N, typename F>
__device__ inline void static_for(F&& f) {
    if constexpr (J < N) {
        f(std::integral_constant<int, J>{});
        static_for<J + 1, N>(f);
    }
}

// Dot chunk C of a super-chunk and accumulate: acc[rg][ct][r] is row
// 4*tq + r of row group rg for slot 16*ct + (lane & 15); ws[rg] holds the
// super-chunk's weight scales as load_scales left them, xb the slots'.  Blocks past K (the
// padding of the last super-chunk) hold zero codes and zero scales on both
// sides: their term is fma(0, +0, acc), which returns acc unchanged (acc
// starts at +0 and no term can make it -0), so they need no test.
template <int C, int RG, int CT>
__device__ inline void mfma_chunk(const Chunk<RG, CT>& ch, const uint32_t ws[RG],
                                  const SlotScales<CT>& xb, float acc[RG][CT][4]) {
    uint32_t wd[RG][4];  // row 4*tq + r: block 2c's scale in the low half, 2c+1's in the high
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        wd[rg][0] = chunk_scale<C, 0>(ws[rg]);
        wd[rg][1] = chunk_scale<C, 1>(ws[rg]);
        wd[rg][2] = chunk_scale<C, 2>(ws[rg]);
        wd[rg][3] = chunk_scale<C, 3>(ws[rg]);
    }
    // The (tile, row group) pairs in order, their two MFMAs issued one pair
    // ahead of the scale arithmetic that consumes them, so that a result is
    // never waited for right after its MFMA.  Each accumulator still takes
    // its block-2c term, then its block-2c+1 term.
    constexpr int P = CT * RG;
    const v4i zero = {0, 0, 0, 0};
    v4i S[2][2];
    S[0][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ch.w[0].x, ch.aq[0].x, zero, 0, 0, 0);
    S[0][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ch.w[0].y, ch.aq[0].y, zero, 0, 0, 0);
    static_for<0, P>([&](auto pc) {
        constexpr int p = decltype(pc)::value;
        constexpr int ct = p / RG, rg = p % RG;
        if constexpr (p + 1 < P) {
            constexpr int ct1 = (p + 1) / RG, rg1 = (p + 1) % RG;
            S[(p + 1) & 1][0] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ch.w[rg1].x, ch.aq[ct1].x, zero, 0, 0, 0);
            S[(p + 1) & 1][1] = __builtin_amdgcn_mfma_i32_16x16x32_i8(ch.w[rg1].y, ch.aq[ct1].y, zero, 0, 0, 0);
        }
        const uint32_t dx = xb.template get<C>(ct);
        const _Float16 dx0 = half_bits(dx, 0), dx1 = half_bits(dx, 1);
        const v4i& S0 = S[p & 1][0];
        const v4i& S1 = S[p & 1][1];
        float* a = acc[rg][ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = term_fma(S0[r], half_bits(wd[rg][r], 0), dx0, a[r]);
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = term_fma(S1[r], half_bits(wd[rg][r], 1), dx1, a[r]);
    });
}

// Loads and stores that are coherent across the whole device (all XCDs)
// without flushing any cache.
__device__ inline float coherent_load(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void coherent_store(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// ------------------------------------------------------------------------
// Fused pre-quantisation.  The first P workgroups of a FUSED launch quantise
// X into the slot buffer (the q8_0 rule of the separate pre-quantiser, same
// bits), write it with device-coherent stores, wait for the stores to
// complete and arrive at the producer counter (two levels, see arrive_last);
// the last of them raises the "published" flags.
// The matmul workgroups put their first weight chunks in flight, then wait
// for their flag before their first activation load.  Workgroups are
// dispatched in index order, so the producers are resident or done before
// any matmul workgroup waits, and they wait on nothing themselves.  The wait
// is bounded all the same (max_spins polls): a workgroup whose wait runs out
// writes quiet NaN over all its outputs (a split publishes a NaN partial, so
// the combined rows are NaN too) and counts itself in the workspace's
// timeout word, which the library never clears, so the failure is loud.
// Every workgroup, producer or matmul, finally arrives at an exit counter
// (after waiting for its own stores and atomics to complete); the last of
// all P + n_cons arrivals rearms the counters and flags.  Nothing can touch
// them after that: every producer has raised what it raises and every
// matmul workgroup has stopped polling.
//
// Why the matmul workgroups may read the slots with plain loads after a
// relaxed poll: every dispatch begins with an agent-scope acquire that
// invalidates the L2 of every XCD (the slot buffer lives in ordinary
// coarse-grained memory), so no line of the slot buffer cached by an
// earlier kernel survives into this one; within the launch no workgroup
// loads a slot line before its flag reads 1 (the loads are issued after the
// poll, behind a workgroup barrier, and are not speculated), and the flag is
// raised only after every producer's device-coherent stores have completed.
// Every slot line that enters any cache during the launch therefore holds
// the published bytes.
// ------------------------------------------------------------------------

// The "published" signal is polled by one thread per workgroup, each on one
// of kReadyCopies flags that sit in different memory pages (4 KB apart), so
// that the polls of a large grid do not all queue on one memory channel.
constexpr int kReadyCopies = 15;
constexpr int kReadyStride = 1024;  // uint32 elements (4 KB)
// Arrivals are counted in two levels: member id of n bumps counter id % 8,
// the last of each of those bumps the top counter.  Atomics on one address
// queue one behind the other at the memory side, so 1000 workgroups on one
// counter take microseconds; 8 counters in different lines share the load.
constexpr int kSubCounters = 8;
constexpr int kSubStride = 32;  // uint32 elements (128 bytes)

// True for the last of the n arrivals (ids 0 .. n-1, each arriving once).
__device__ inline bool arrive_last(uint32_t* top, uint32_t* sub, int id, int n) {
    const int s = id % kSubCounters;
    const int groups = n < kSubCounters ? n : kSubCounters;
    const uint32_t in_group = (uint32_t)((n - s + kSubCounters - 1) / kSubCounters);
    if (__hip_atomic_fetch_add(sub + s * kSubStride, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) !=
        in_group - 1)
        return false;
    return __hip_atomic_fetch_add(top, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (uint32_t)(groups - 1);
}

// Wait until this thread's earlier memory operations (stores and atomics)
// have completed.
__device__ inline void wait_memory() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Called by thread 0 of every workgroup of a FUSED launch, last thing: the
// last of all arrivals rearms every counter and flag for the next call.
__device__ inline void fused_exit(const MmArgs& a) {
    wait_memory();
    if (!arrive_last(a.qexit, a.qexit_sub, (int)blockIdx.x, a.P + a.n_cons)) return;
    __hip_atomic_store(a.qflag, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(a.qexit, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    for (int k = 0; k < kSubCounters; ++k) {
        __hip_atomic_store(a.qflag_sub + k * kSubStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(a.qexit_sub + k * kSubStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int k = 0; k < kReadyCopies; ++k)
        __hip_atomic_store(a.qready + k * kReadyStride, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ void produce_slots(const MmArgs& a, int pid) {
    const int nthreads = blockDim.x;
    const int64_t bpr = (int64_t)a.NSC * kScBlocks;  // blocks per row, padded
    const int64_t total = (int64_t)a.n_rows * bpr * 4;  // one lane per 8 values
    uint8_t* xq = const_cast<uint8_t*>(a.xq);
    uint16_t* xd = const_cast<uint16_t*>(a.xd);
    // strides are multiples of 64 and rows hold an even number of blocks, so
    // a wave always holds whole pairs of blocks (8 lanes) of one row
    for (int64_t tid = (int64_t)pid * nthreads + threadIdx.x; tid < total;
         tid += (int64_t)a.P * nthreads) {
        const int seg = (int)(tid & 3);
        const int64_t b = tid >> 2;
        const int64_t blk = b % bpr, row = b / bpr;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (blk < a.KB) {
            const float* p = a.X + row * ((int64_t)a.KB * kBlock) + blk * kBlock + seg * 8;
            const float4 x0 = *reinterpret_cast<const float4*>(p);
            const float4 x1 = *reinterpret_cast<const float4*>(p + 4);
            v[0] = x0.x; v[1] = x0.y; v[2] = x0.z; v[3] = x0.w;
            v[4] = x1.x; v[5] = x1.y; v[6] = x1.z; v[7] = x1.w;
        }
        const QuantSeg r = quantize_segment(v);
        const uint64_t q = (uint64_t)r.lo | ((uint64_t)r.hi << 32);
        __hip_atomic_store(reinterpret_cast<uint64_t*>(xq + packed_q_offset(row, blk, seg, a.NSC)), q,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // the odd block's scale sits next to the even block's: one 4-byte store
        const uint32_t d_next = __shfl_down((uint32_t)r.d16, 4);
        if (seg == 0 && (blk & 1) == 0)
            __hip_atomic_store(reinterpret_cast<uint32_t*>(xd + packed_d_index(row, blk, a.NSC)),
                               (uint32_t)r.d16 | (d_next << 16), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    wait_memory();
    __syncthreads();
    if (threadIdx.x == 0) {
        if (arrive_last(a.qflag, a.qflag_sub, pid, a.P)) {
            // the last producer: every slot is published; raise all the flags
            for (int k = 0; k < kReadyCopies; ++k)
                __hip_atomic_store(a.qready + k * kReadyStride, 1u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        fused_exit(a);
    }
}

// Called by every thread of a matmul workgroup: thread 0 polls the
// workgroup's flag, at most a.max_spins times, the others wait at the
// barriers.  Returns true (in every thread) if the wait ran out; thread 0
// has then counted the workgroup in the timeout word.
__device__ inline bool wait_for_slots(const MmArgs& a, int bid, int* shared_flag) {
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t* f = a.qready + (bid % kReadyCopies) * kReadyStride;
        int ready = 0;
        for (int spins = 0; spins < a.max_spins; ++spins) {
            if (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
                ready = 1;
                break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        if (!ready)
            __hip_atomic_fetch_add(a.timeouts, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *shared_flag = !ready;
    }
    __syncthreads();
    return *shared_flag != 0;
}

// An output unit is 4 consecutive rows of one row group for one token: unit
// v of the n_live x RG x 4 units of a tile is token v / (4 RG), row group
// (v / 4) % RG, rows 4 (v % 4) .. +3.  Consecutive threads take consecutive
// units, so four threads store a token's 16 rows of a row group (64
// contiguous bytes).  Rows past N and row groups before gskip (owned by the
// previous row block) are not stored.
template <int RG>
__device__ inline void store_unit(const MmArgs& a, int v, int64_t gbase, int gskip, float4 y) {
    const int t = v / (4 * RG), rg = (v >> 2) & (RG - 1), q = v & 3;
    if (rg < gskip) return;
    const int64_t n0 = (gbase + rg) * kRowsPerGroup + 4 * q;
    float* yrow = a.Y + (int64_t)t * a.N;
    if (a.y_vec4 && n0 + 3 < a.N) {
        *reinterpret_cast<float4*>(yrow + n0) = y;
    } else {
        if (n0 < a.N) yrow[n0] = y.x;
        if (n0 + 1 < a.N) yrow[n0 + 1] = y.y;
        if (n0 + 2 < a.N) yrow[n0 + 2] = y.z;
        if (n0 + 3 < a.N) yrow[n0 + 3] = y.w;
    }
}

__device__ inline float4 add4(float4 p, float4 q) {
    return make_float4(p.x + q.x, p.y + q.y, p.z + q.z, p.w + q.w);
}

// The sums of this thread's units over the NW waves of the workgroup, in the
// tree's order: waves in order within a split, splits (of KW waves each) in
// order.  red4 holds the waves' partial tiles as [wave][rg][slot][4 rows]
// float4s; col[i] is unit i's slot column.  NW is a template parameter so
// that every LDS read of a unit is issued before any add, with no branch.
template <int NW, int RG, int SL, int MU>
__device__ inline void tile_sums(const float4* red4, const int col[MU], int nthreads, int S,
                                 int KW, float4 y[MU]) {
#pragma unroll
    for (int i = 0; i < MU; ++i) {
        const int v = threadIdx.x + i * nthreads;  // units past the live ones are computed and dropped
        const int rg = (v >> 2) & (RG - 1), q = v & 3;
        float4 p[NW];
#pragma unroll
        for (int k = 0; k < NW; ++k) p[k] = red4[((k * RG + rg) * SL + col[i]) * 4 + q];
        float4 sum = p[0];
        if (S == 1 || KW == 1) {  // one level: the waves in order
#pragma unroll
            for (int k = 1; k < NW; ++k) sum = add4(sum, p[k]);
        } else {  // each split's waves in order, then the splits in order
            float4 part = p[0];
#pragma unroll
            for (int k = 1; k < NW; ++k) {
                if (k % KW == 0) {
                    sum = (k == KW) ? part : add4(sum, part);
                    part = p[k];
                } else {
                    part = add4(part, p[k]);
                }
            }
            sum = add4(sum, part);
        }
        y[i] = sum;
    }
}

// Level 2 of the tree by the last of the NS splits of a row block to arrive:
// its units' partials of the other splits come from the workspace
// (device-coherent loads, all issued before any is added), its own from
// registers; they are added in split order and Y is stored.
template <int NS, int RG, int MU>
__device__ inline void combine_splits(const MmArgs& a, int rec, int split, int E, int nthreads,
                                      int U, const float4 y[MU], const bool bad[MU],
                                      int64_t gbase, int gskip) {
#pragma unroll
    for (int i = 0; i < MU; ++i) {
        const int v = threadIdx.x + i * nthreads;
        if (v >= U) continue;
        float4 p[NS];
#pragma unroll
        for (int sp = 0; sp < NS; ++sp) {
            if (sp == split) continue;
            const float* part = record_part(a.recs, rec, NS, E, sp) + v;
            p[sp] = make_float4(coherent_load(part), coherent_load(part + E / 4),
                                coherent_load(part + E / 2), coherent_load(part + 3 * (E / 4)));
        }
#pragma unroll
        for (int sp = 0; sp < NS; ++sp)
            if (sp == split) p[sp] = y[i];
        float4 sum = p[0];
#pragma unroll
        for (int sp = 1; sp < NS; ++sp) sum = add4(sum, p[sp]);
        const float nan = __builtin_nanf("");
        store_unit<RG>(a, v, gbase, gskip, bad[i] ? make_float4(nan, nan, nan, nan) : sum);
    }
}

// One workgroup per row block (plain: all S*KW waves; WHOLE: one wave that
// takes the S splits in turn) or per (row block, split) (SPLIT: KW waves;
// with WHOLE, the first n_whole row blocks run as whole workgroups and only
// the rest as splits).  LDS: the wave partials red, fp32, one float4 per
// lane and (row group, column tile) of each wave.
// FUSED: the first P workgroups are producers (see above).
template <int RG, int CT, int D, bool NTW, bool SPLIT, bool FUSED, bool WHOLE>
__global__ void __launch_bounds__(512)
mm_mfma_kernel(MmArgs a) {
    int bid = (int)blockIdx.x;
    if (FUSED) {
        if (bid < a.P) {
            produce_slots(a, bid);
            return;
        }
        bid -= a.P;
    }
    WaveStamps st;
    static_assert(D == 1 || D == 2 || D == 4, "the ring depth must divide a super-chunk");
    static_assert(RG == 1 || RG == 2 || RG == 4, "row groups per wave");
    extern __shared__ __align__(16) float red[];
    __shared__ int wait_expired;
    __shared__ int last_split;
    static_assert(CT >= 1 && CT * 16 <= kMaxColumns, "column tiles");
    constexpr int E = RG * CT * 256;  // output tile: RG row groups x 16 rows x 16*CT slots
    const int lane = threadIdx.x & 63;
    const int tq = lane >> 4;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    // A whole workgroup (the first n_whole row blocks) is one wave that
    // streams its row block's whole rows and evaluates the S splits in turn:
    // at each split's first super-chunk it folds the partial so far (the
    // tree's level 2, in split order) and starts the next from zero, so its
    // sums are those of S separate split waves.  A SPLIT launch runs the row
    // blocks after those as S one-split workgroups each.  Only the WHOLE
    // kernels (one row group per wave, launched when n_whole > 0) carry the
    // code; the others are unchanged by it.
    static_assert(!WHOLE || RG == 1, "whole workgroups stream one row group");
    const int n_whole = WHOLE ? a.n_whole : 0;
    const bool whole = WHOLE && bid < n_whole;
    const int nwaves = (SPLIT || WHOLE) ? a.KW : a.S * a.KW;
    const int piece = SPLIT && !whole ? bid - n_whole : 0;
    const int rb = SPLIT && !whole ? n_whole + piece / a.S : bid;
    const int split = whole ? 0 : SPLIT ? piece % a.S : w / a.KW;
    int sc0 = 0, sc1 = a.NSC;
    if (!whole) slice_range(a.NSC, a.S, a.KW, split, SPLIT ? w : w % a.KW, sc0, sc1);
    const int c_lo = 4 * sc0;  // this wave's chunks: [c_lo, 4 * sc1), at least one super-chunk

    // weights: RG consecutive row groups; the last row block may start
    // earlier (gbase < g0) so that every load stays inside the buffer, and
    // then stores only the groups from g0 on
    const int64_t g0 = (int64_t)rb * RG;
    const int64_t gbase = min(g0, a.G - RG);
    const int64_t gq = (int64_t)a.NSC * kScQBytes;              // bytes per row group
    const int64_t gd = (int64_t)a.NSC * 4 * (kChunkDBytes / 2);  // halves per row group
    // this lane's scale dword of a super-chunk: row 4*tq + (j & 3) of chunk j >> 2
    const int jl = lane & 15;
    constexpr bool BUF = CT >= 2;
    const auto wrow = operand<BUF>(a.wq + gbase * gq, (a.G - gbase) * gq, lane * 16);
    const auto wsrow = operand<BUF>(a.wd + gbase * gd, (a.G - gbase) * gd,
                                    ((jl >> 2) * kRowsPerGroup + 4 * tq + (jl & 3)) * 2);
    const auto xa = operand<BUF>(a.xq, a.CT * a.xq_gs, lane * 16);
    const auto xsrow = operand<BUF>(a.xd, a.CT * a.xd_gs, lane * 2);
    const int gskip = (int)(g0 - gbase);

    float acc[RG][CT][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[rg][ct][r] = 0.0f;
    // a whole wave's level 2: the splits folded so far, and the super-chunk
    // where the next split starts
    float tot[RG][CT][4];
    int fold_s = 1;
    int fold_at = whole && a.S > 1 ? a.NSC / a.S : a.NSC;
    auto fold = [&]() {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    tot[rg][ct][r] = fold_s == 1 ? acc[rg][ct][r] : tot[rg][ct][r] + acc[rg][ct][r];
                    acc[rg][ct][r] = 0.0f;
                }
        ++fold_s;
        fold_at = fold_s < a.S ? fold_s * a.NSC / a.S : a.NSC;
    };

    // the live tokens' slots, for the output gather: lane t of each wave
    // holds batch_index[t], read now so that the load's latency hides behind
    // the weight stream
    int my_slot = 0;
    if (lane < a.n_live) my_slot = a.bidx[lane];

    // The ring: chunk c sits in ring[c % D].  The scales of the next
    // super-chunk are loaded just before the first chunk of it, so waiting for
    // that chunk covers them too.
    Chunk<RG, CT> ring[D];
    uint32_t ws_next[RG], xs_next[CT];
    load_scales<RG>(ws_next, sc0, wsrow, gd);
    bool poison = false;
    if (FUSED) {
        // weights first; the slots only once the producers have published them
#pragma unroll
        for (int i = 0; i < D; ++i) load_chunk_w<RG, CT, NTW>(ring[i], c_lo + i, wrow, gq);
        poison = wait_for_slots(a, bid, &wait_expired);
        load_slot_scales<CT>(xs_next, sc0, xsrow, a.xd_gs);
#pragma unroll
        for (int i = 0; i < D; ++i) load_chunk_a<RG, CT>(ring[i], c_lo + i, xa, a.xq_gs);
    } else if constexpr (BUF) {
        // in ring order (the barriers keep them so): the loop's first wait is
        // then for the oldest loads only; left alone, the scheduler may issue
        // ring[0] last, and the first wait is for all of them
        load_slot_scales<CT>(xs_next, sc0, xsrow, a.xd_gs);
        __builtin_amdgcn_sched_barrier(0);
        static_for<0, D>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            load_chunk<RG, CT, NTW>(ring[i], c_lo + i, wrow, gq, xa, a.xq_gs);
            __builtin_amdgcn_sched_barrier(0);
        });
    } else {
        load_slot_scales<CT>(xs_next, sc0, xsrow, a.xd_gs);
#pragma unroll
        for (int i = 0; i < D; ++i) load_chunk<RG, CT, NTW>(ring[i], c_lo + i, wrow, gq, xa, a.xq_gs);
    }
    int sc = sc0;
    SlotScales<CT> xb;
    // All super-chunks but the last, in runs that end where a whole wave
    // folds (between runs, never inside the loop body: a test there is
    // if-converted into selects on every accumulator, every turn).
    for (;;) {
        const int run_end = whole && fold_at < sc1 - 1 ? fold_at : sc1 - 1;
        for (; sc < run_end; ++sc) {
            uint32_t ws[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) ws[rg] = ws_next[rg];
            xb.prepare(xs_next);
            static_for<0, 4>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                mfma_chunk<j, RG, CT>(ring[j % D], ws, xb, acc);
                if constexpr (j == 0) st.mark_once(1);
                // Two-row-group buffer kernels: nor above the dot (only VALU and
                // SALU work may cross).  Their ring is near the register limit,
                // and loads hoisted above the dot need a spare ring slot: the
                // 4-tile one then spills.
                if constexpr (BUF && RG >= 2) __builtin_amdgcn_sched_barrier(0x6);
                if constexpr ((j + D) % 4 == 0) {
                    load_scales<RG>(ws_next, sc + 1, wsrow, gd);
                    load_slot_scales<CT>(xs_next, sc + 1, xsrow, a.xd_gs);
                }
                load_chunk<RG, CT, NTW>(ring[j % D], 4 * sc + j + D, wrow, gq, xa, a.xq_gs);
                // keep each chunk's loads right after its dot: left alone, the
                // scheduler sinks all the chunks' loads to the end of the turn,
                // and every turn then waits a full memory latency
                __builtin_amdgcn_sched_barrier(0);
            });
        }
        if (!whole || sc >= sc1 - 1) break;
        fold();  // sc is the next split's first super-chunk
    }
    // the last super-chunk: its chunks are in the ring or loaded here
    if (whole && sc == fold_at) fold();
    xb.prepare(xs_next);
    static_for<0, 4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        mfma_chunk<j, RG, CT>(ring[j % D], ws_next, xb, acc);
        if constexpr (j == 0) st.mark_once(1);
        if constexpr (j + D < 4)
            load_chunk<RG, CT, NTW>(ring[j % D], 4 * sc + j + D, wrow, gq, xa, a.xq_gs);
    });

    if (whole && a.S > 1) {  // the last split's partial joins the folded ones
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rg][ct][r] = tot[rg][ct][r] + acc[rg][ct][r];
    }
    st.mark(2);
    // Epilogue.  Every wave writes its partial tile to LDS as [wave][row
    // group][slot][16 rows] (lane (tq, j) writes rows 4tq .. 4tq+3 of slot
    // 16ct + j as one float4); then each thread takes whole output units (see
    // store_unit), reads its token's slot column of every wave's tile (all
    // the reads issued before any add) and adds them in the tree's order:
    // waves in order within a split, splits in order.
    constexpr int SL = 16 * CT;  // slot columns
    constexpr int MU = RG * CT;  // units per thread at most (n_live <= SL, >= 64 threads)
    float4* red4 = reinterpret_cast<float4*>(red);
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            red4[((w * RG + rg) * SL + ct * 16 + (lane & 15)) * 4 + tq] =
                make_float4(acc[rg][ct][0], acc[rg][ct][1], acc[rg][ct][2], acc[rg][ct][3]);
    __syncthreads();
    st.mark(3);
    if (FUSED && threadIdx.x == 0) fused_exit(a);
    const int nthreads = nwaves * 64;
    const int U = a.n_live * RG * 4;
    // this thread's units, their slot columns (lane t of every wave holds
    // batch_index[t]; the shuffle runs in every lane) and the tree's sums
    // over this workgroup's waves
    int col[MU];
    bool bad[MU];
    float4 y[MU];
#pragma unroll
    for (int i = 0; i < MU; ++i) {
        const int v = threadIdx.x + i * nthreads;
        const int t = v < U ? v / (4 * RG) : 0;
        const int sl = __shfl(my_slot, t);
        bad[i] = poison || sl < 0 || sl >= SL;
        col[i] = bad[i] ? 0 : sl;
    }
    {
        // a split or whole workgroup sums its KW waves only
        const int S_here = (SPLIT || whole) ? 1 : a.S;
        switch (nwaves) {
#define Q8_SUMS(NW) \
            case NW: tile_sums<NW, RG, SL, MU>(red4, col, nthreads, S_here, a.KW, y); break;
            Q8_SUMS(1) Q8_SUMS(2) Q8_SUMS(3) Q8_SUMS(4) Q8_SUMS(5) Q8_SUMS(6) Q8_SUMS(7) Q8_SUMS(8)
#undef Q8_SUMS
            default: break;  // more waves than a workgroup may hold: never launched
        }
    }
    if (!SPLIT || whole) {
#pragma unroll
        for (int i = 0; i < MU; ++i) {
            const int v = threadIdx.x + i * nthreads;
            if (v < U) {
                const float nan = __builtin_nanf("");
                store_unit<RG>(a, v, gbase, gskip, bad[i] ? make_float4(nan, nan, nan, nan) : y[i]);
            }
        }
        st.mark(4);
        st.drain();
        st.mark(5);
        st.write(a, (int64_t)bid * nwaves + w, lane);
        return;
    }
    // Level 2 across workgroups.  This split's units go to the workspace
    // with device-coherent stores, component-major (component c of unit v at
    // float c*E/4 + v: each store instruction then covers whole cache lines,
    // where a unit-major layout sends every line through four partial
    // writes); once every thread's stores have completed, the split arrives
    // at its row block's counter.  The last to arrive loads the other
    // splits' units (device-coherent loads, all issued before any is added),
    // adds the S partials in split order, its own straight from registers,
    // stores Y and rearms the counter.
    static_assert(!SPLIT || CT == 1, "split execution has one column tile");
    static_assert(kMaxSlots * RG * 4 <= E / 4, "a component block holds every unit");
    const int rec = rb - n_whole;  // records cover the split row blocks only
    float* mine = record_part(a.recs, rec, a.S, E, split);
#pragma unroll
    for (int i = 0; i < MU; ++i) {
        const int v = threadIdx.x + i * nthreads;
        if (v < U) {
            // a workgroup whose wait ran out publishes NaN: the combined rows are NaN
            const float4 o = bad[i] ? make_float4(__builtin_nanf(""), __builtin_nanf(""),
                                                  __builtin_nanf(""), __builtin_nanf(""))
                                    : y[i];
            coherent_store(mine + v, o.x);
            coherent_store(mine + E / 4 + v, o.y);
            coherent_store(mine + E / 2 + v, o.z);
            coherent_store(mine + 3 * (E / 4) + v, o.w);
        }
    }
    wait_memory();
    __syncthreads();
    st.mark(4);
    if (threadIdx.x == 0)
        last_split = __hip_atomic_fetch_add(record_counter(a.recs, rec, a.S, E), 1u,
                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                     (uint32_t)(a.S - 1);
    __syncthreads();
    st.mark(5);
    if (!last_split) {
        st.write(a, (int64_t)bid * nwaves + w, lane);
        return;
    }
    switch (a.S) {
#define Q8_COMBINE(NS) \
        case NS: combine_splits<NS, RG, MU>(a, rec, split, E, nthreads, U, y, bad, gbase, gskip); break;
        Q8_COMBINE(2) Q8_COMBINE(3) Q8_COMBINE(4) Q8_COMBINE(5) Q8_COMBINE(6) Q8_COMBINE(7)
        Q8_COMBINE(8)
#undef Q8_COMBINE
        default: break;  // more splits than the tiling makes: never launched
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(record_counter(a.recs, rec, a.S, E), 0u, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    st.drain();
    st.mark(6);
    st.write(a, (int64_t)bid * nwaves + w, lane);
}

int mfma_waves(const MmArgs& a, bool split) {
    return (split || a.n_whole > 0) ? a.KW : a.S * a.KW;
}

size_t mfma_lds_bytes(const MmArgs& a, int rg, int ct, bool split) {
    return (size_t)mfma_waves(a, split) * rg * ct * 256 * sizeof(float);
}

int mfma_max_waves(int) { return 8; }  // 512 threads: 256 VGPRs per lane

template <int RG, int CT, int D, bool NTW, bool SPLIT, bool FUSED = false, bool WHOLE = false>
hipError_t launch_mfma(MmArgs a, hipStream_t st) {
    const int waves = mfma_waves(a, SPLIT);
    const size_t lds = mfma_lds_bytes(a, RG, CT, SPLIT);
    if (lds > kMaxLds || waves > mfma_max_waves(RG) || a.G < RG || a.CT != CT)
        return hipErrorInvalidValue;
    if (a.n_whole < 0 || a.n_whole > a.n_rb || (a.n_whole > 0) != WHOLE ||
        (WHOLE && a.KW != 1) || (!SPLIT && a.n_whole != 0 && a.n_whole != a.n_rb))
        return hipErrorInvalidValue;
    const int64_t cons = SPLIT ? a.n_whole + (int64_t)(a.n_rb - a.n_whole) * a.S : a.n_rb;
    int64_t grid = cons;
    if (FUSED) {
        // producers: one lane per 8 activation values, 64*waves lanes each
        // (none when the caller asked for no quantisation: a P of 0)
        const int64_t lanes = (int64_t)a.n_rows * a.NSC * kScBlocks * 4;
        if (a.P != 0) a.P = (int)((lanes + 64 * waves - 1) / (64 * waves));
        a.n_cons = (int)cons;
        grid += a.P;
    }
    hipLaunchKernelGGL((mm_mfma_kernel<RG, CT, D, NTW, SPLIT, FUSED, WHOLE>), dim3((unsigned)grid),
                       dim3(64 * waves), lds, st, a);
    return hipGetLastError();
}

// ------------------------------------------------------------------------
// DOT4 engine: one row per lane, 64 rows (4 row groups) per wave.
// ------------------------------------------------------------------------

template <int NT, bool TAIL>
__device__ inline void dot4_step(int sc, int nb, const uint8_t* wrow,
                                 const uint16_t* wdrow, const MmArgs& a,
                                 const int slot[NT], float acc[NT]) {
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
        if (TAIL && 2 * c >= nb) break;
        const int64_t chunk = (int64_t)sc * 4 + c;
        uint4 w[4];  // [k-slot]: this row's 8 bytes of blocks 2c and 2c+1
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = ld16(wrow + chunk * kChunkBytes + k * 256);
        const uint32_t wdc = *reinterpret_cast<const uint32_t*>(wdrow + chunk * (kChunkDBytes / 2));
        const _Float16 dw0 = half_bits(wdc, 0), dw1 = half_bits(wdc, 1);
        const bool has1 = !TAIL || 2 * c + 1 < nb;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const uint8_t* xs = a.xq + chunk * kChunkBytes + slot[t] * 16;
            int S0 = 0, S1 = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const u32x4 x = *(cu32x4*)(xs + k * 256);
                S0 = __builtin_amdgcn_sdot4((int)w[k].x, (int)x.x, S0, false);
                S0 = __builtin_amdgcn_sdot4((int)w[k].y, (int)x.y, S0, false);
                S1 = __builtin_amdgcn_sdot4((int)w[k].z, (int)x.z, S1, false);
                S1 = __builtin_amdgcn_sdot4((int)w[k].w, (int)x.w, S1, false);
            }
            const uint32_t dv = *(const __attribute__((address_space(4))) uint32_t*)(
                a.xd + (chunk * 16 + slot[t]) * 2);
            acc[t] = term_fma(S0, dw0, half_bits(dv, 0), acc[t]);
            if (has1) acc[t] = term_fma(S1, dw1, half_bits(dv, 1), acc[t]);
        }
    }
}

template <int NT>
__global__ void __launch_bounds__(1024)
mm_dot4_kernel(MmArgs a) {
    extern __shared__ float red[];  // wave partials [S*KW][NT*64]
    constexpr int E = NT * 64;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int nwaves = a.S * a.KW;
    int sc0, sc1;
    slice_range(a.NSC, a.S, a.KW, w / a.KW, w % a.KW, sc0, sc1);
    const int64_t g0 = (int64_t)blockIdx.x * 4;
    const int64_t g = min(g0 + (lane >> 4), a.G - 1);
    const int j = lane & 15;
    const uint8_t* wrow = a.wq + g * a.NSC * kScQBytes + j * 16;
    const uint16_t* wdrow = a.wd + g * a.NSC * 4 * (kChunkDBytes / 2) + j * 2;
    int slot[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) slot[t] = __builtin_amdgcn_readfirstlane(live_slot(a.bidx, a.n_live, t));
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;

    const int sc_full = min(sc1, a.KB / kScBlocks);
    int sc = sc0;
    for (; sc < sc_full; ++sc) dot4_step<NT, false>(sc, kScBlocks, wrow, wdrow, a, slot, acc);
    if (sc < sc1) dot4_step<NT, true>(sc, a.KB - sc * kScBlocks, wrow, wdrow, a, slot, acc);

#pragma unroll
    for (int t = 0; t < NT; ++t) red[w * E + t * 64 + lane] = acc[t];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += nwaves * 64) {
        const float y = tree_sum(red, E, e, a.S, a.KW);
        const int t = e >> 6, ln = e & 63;
        const int64_t nn = (g0 + (ln >> 4)) * kRowsPerGroup + (ln & 15);
        if (nn < a.N) a.Y[(int64_t)t * a.N + nn] = slot_bad(a.bidx, t) ? __builtin_nanf("") : y;
    }
}

template <int NT>
hipError_t launch_dot4_nt(const MmArgs& a, hipStream_t st) {
    const unsigned grid = (unsigned)((a.G + 3) / 4);
    const int waves = a.S * a.KW;
    if (waves > kMaxKs) return hipErrorInvalidValue;
    const size_t lds = (size_t)waves * NT * 64 * sizeof(float);
    hipLaunchKernelGGL(mm_dot4_kernel<NT>, dim3(grid), dim3(64 * waves), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_dot4(const MmArgs& a, hipStream_t st) {
    switch (a.n_live) {
        case 1: return launch_dot4_nt<1>(a, st);
        case 2: return launch_dot4_nt<2>(a, st);
        case 3: return launch_dot4_nt<3>(a, st);
        case 4: return launch_dot4_nt<4>(a, st);
        case 5: return launch_dot4_nt<5>(a, st);
        case 6: return launch_dot4_nt<6>(a, st);
        case 7: return launch_dot4_nt<7>(a, st);
        case 8: return launch_dot4_nt<8>(a, st);
        case 9: return launch_dot4_nt<9>(a, st);
        case 10: return launch_dot4_nt<10>(a, st);
        case 11: return launch_dot4_nt<11>(a, st);
        case 12: return launch_dot4_nt<12>(a, st);
        case 13: return launch_dot4_nt<13>(a, st);
        case 14: return launch_dot4_nt<14>(a, st);
        case 15: return launch_dot4_nt<15>(a, st);
        case 16: return launch_dot4_nt<16>(a, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

// Weights in flight over the whole GPU at which the stream runs fastest
// (measured on MI355X; see choose_tiling).
constexpr int64_t kInFlightKB = 4400;

Tiling choose_tiling(const Shape& s) {
    // Rules measured on MI355X over the model-shaped matrices (K 5120..18432,
    // N 5120..151936):
    //  * two row groups per wave (each activation load feeds 32 rows);
    //  * long rows (K >= 8192) are cut into 4 splits of one wave each, which
    //    the workspace entry point runs as separate single-row-group
    //    workgroups (more of them than there are CUs), 4 chunks in flight
    //    per wave; when the two-row-group blocks number 205..256 (at least
    //    80% of the CUs, one each), as 4 wave slices of one workgroup;
    //  * shorter rows are one split.  Below 1024 row groups (16k rows) it is
    //    two row groups per wave and 4 wave slices per row block, 4 chunks
    //    in flight each.  From 1024 row groups on, the weight stream runs
    //    fastest with about kInFlightKB of weights in flight over the whole
    //    GPU (more outstanding requests lower the rate HBM delivers): one
    //    wave per row group, covering the whole row, with the ring depth
    //    (4, 2 or 1 chunks) that comes closest, e.g. 7168->18432 at 4,
    //    gate+up 5120->34816 at 2.  Past kInFlightKB row groups even depth 1
    //    is too much: two row groups per wave then halve the waves (a
    //    152k-row head);
    //  * never more wave slices than super-chunks;
    //  * one wave per row group leaves the CUs unevenly loaded when the row
    //    groups are not a multiple of the 256 CUs: with gate+up's 2176, 128
    //    CUs stream 9 row groups and 128 stream 8, and the kernel lasts as
    //    long as the 9.  Then the tree has S = min(4, 256 / r, NSC) splits
    //    (r = G mod 256, S >= 2; 4 for r = 128) and the split execution runs the first
    //    G - r row groups as one wave each that evaluates the splits in turn
    //    and only the last r as S one-split workgroups each: at most one
    //    piece per CU, dispatched after the whole rows.  Every other
    //    execution evaluates the same splits in one wave per row group.
    constexpr int64_t kCUs = 256;  // MI355X compute units
    Tiling t;
    t.rg = s.G >= 2 ? 2 : 1;
    t.ring = 4;
    t.seq = false;
    t.split_from = 0;
    if (s.NSC >= 32) {
        const int64_t blocks2 = (s.G + 1) / 2;  // two-row-group row blocks
        if (s.G >= 2 && 5 * blocks2 >= 4 * kCUs && blocks2 <= kCUs) {
            // they fill at least 80% of the CUs, one each: the 4 K ranges
            // are 4 wave slices of one workgroup, summed in LDS (the same
            // ranges in the same order as 4 splits, so the same bits), and
            // no workspace: 18432->7168 (224 row blocks) 24.6 against 25.0-25.1 us
            t.splits = 1;
            t.kw = 4;
            t.rg_split = 2;
        } else {
            t.splits = 4;
            t.kw = 1;
            t.rg_split = 1;
        }
    } else {
        t.splits = 1;
        int64_t kw = 4;
        if (s.G >= 1024) {
            kw = 1;
            if (s.G <= kInFlightKB) {
                t.rg = 1;
                t.ring = 3 * s.G <= kInFlightKB ? 4 : 3 * s.G <= 2 * kInFlightKB ? 2 : 1;
                const int64_t r = s.G % kCUs;
                int64_t st = r == 0 ? 1 : std::min<int64_t>({4, kCUs / r, s.NSC});
                // r = 128: 4 splits put exactly two quarter-row pieces on
                // every CU, as even as one half-row piece, and give the
                // multi-column launches (one wave per split) twice the
                // waves: 7168->18432 at 64 columns 51.5 -> 44.7 us, the
                // one-column kernels unchanged
                if (2 * r == kCUs && s.NSC >= 4) st = 4;
                if (st >= 2) {
                    t.splits = (int)st;
                    t.seq = true;
                    t.split_from = s.G - r;
                }
            } else {
                t.ring = 1;
            }
        }
        t.rg_split = t.rg;
        t.kw = (int)std::min<int64_t>(kw, s.NSC);
    }
    t.nt_weights = true;
    return t;
}

// Row groups per wave actually launched (a matrix with fewer row groups than
// asked for runs one per wave).
// The one-tile (16-slot) kernels: row groups per wave, split or not, and
// ring depth as the tiling asks.
template <bool FUSED>
hipError_t launch_ct1(const MmArgs& a, int rg, bool split, int ring, bool nt_weights,
                      hipStream_t st) {
#define Q8_CT1(R, D)                                                               \
    if (rg == R && ring == D && a.n_whole == 0)                                    \
        return split ? launch_mfma<R, 1, D, true, true, FUSED>(a, st)              \
                     : launch_mfma<R, 1, D, true, false, FUSED>(a, st);
#define Q8_CT1_WHOLE(D)                                                            \
    if (rg == 1 && ring == D && a.n_whole > 0)                                     \
        return split ? launch_mfma<1, 1, D, true, true, FUSED, true>(a, st)        \
                     : launch_mfma<1, 1, D, true, false, FUSED, true>(a, st);
    (void)nt_weights;
    Q8_CT1(2, 4) Q8_CT1(2, 1) Q8_CT1(1, 4) Q8_CT1(1, 2) Q8_CT1(1, 1)
    Q8_CT1_WHOLE(4) Q8_CT1_WHOLE(2) Q8_CT1_WHOLE(1)
#undef Q8_CT1_WHOLE
#undef Q8_CT1
    return hipErrorInvalidValue;
}

int launch_rg(const Shape& s, const Tiling& t, bool split) {
    const int rg = split ? t.rg_split : t.rg;
    return s.G >= rg ? rg : 1;
}

size_t workspace_bytes(const Shape& s, const Tiling& t) {
    if (t.splits <= 1) return 0;
    const int rg = launch_rg(s, t, true);
    const int64_t n_rb = (s.G + rg - 1) / rg - t.split_from / rg;  // split row blocks
    return (size_t)(n_rb * record_bytes(t.splits, rg * 256));
}

bool plan_matmul(const Shape& s, const Tiling& t, int n_slots, bool with_workspace,
                 MmPlan& p) {
    p.ct = n_slots / kMaxSlots;
    if (p.ct < 1 || p.ct * kMaxSlots != n_slots || n_slots > kMaxColumns) return false;
    if (t.splits * t.kw > s.NSC) return false;
    p.splits = t.splits;
    p.kw = t.kw;
    p.split = with_workspace && t.splits > 1;
    if (p.split && p.ct != 1) return false;
    if (p.ct == 1) {
        p.rg = launch_rg(s, t, p.split);
        p.ring = t.ring;
        if (t.split_from % p.rg != 0) return false;
        p.n_rb = (int)((s.G + p.rg - 1) / p.rg);
        p.n_whole = p.split ? (int)(t.split_from / p.rg) : t.seq ? p.n_rb : 0;
    } else {
        // More than one column tile: two row groups per wave (one only for a
        // single row group), so each chunk's activation operand (16 bytes per
        // lane and column tile) feeds 32 rows, and the S * KW waves of a row
        // block evaluate the tree's splits and slices side by side, the same
        // sums as every other execution.  Measured on MI355X, same bits: gate+up
        // 5120->34816 at 64 columns 66.0 -> 58.1 us against one row group per
        // whole-row wave, the 152k-row head 263 -> 204.5 us (at 32 columns
        // 194 -> 149 us).  The ring depth keeps the weights in flight over the
        // GPU (one KB per row group and chunk) near what each tile width runs
        // best with: two tiles at most 2 * kInFlightKB at depth 4, 2 or 1 (4
        // whenever a row is cut into 4 or more wave slices: short waves need the
        // depth, gate+up at 32 columns 40.4 us at 4, 41.7 at 1); four
        // tiles at most 2.5 * kInFlightKB at depth 4, else 2 (at depth 1 a
        // wave's four tiles of arithmetic stall on every chunk); three tiles
        // hold 2 chunks in registers.
        p.rg = s.G >= 2 ? 2 : 1;
        p.n_rb = (int)((s.G + p.rg - 1) / p.rg);
        p.n_whole = 0;
        const int64_t kb = (int64_t)p.n_rb * t.splits * t.kw * p.rg;  // KB per chunk of every wave
        const int d2 = (4 * kb <= 2 * kInFlightKB || t.splits * t.kw >= 4) ? 4
                     : 2 * kb <= 2 * kInFlightKB ? 2 : 1;
        const int d4 = 8 * kb <= 5 * kInFlightKB ? 4 : 2;
        p.ring = p.rg == 1 || p.ct == 3 ? 2 : p.ct == 2 ? d2 : d4;
    }
    p.waves = (p.split || p.n_whole > 0) ? t.kw : t.splits * t.kw;
    p.workgroups = p.split ? p.n_whole + (int64_t)(p.n_rb - p.n_whole) * t.splits : p.n_rb;
    p.lds_bytes = (size_t)p.waves * p.rg * p.ct * 256 * sizeof(float);
    return true;
}

#ifdef Q8_TIMELINE
namespace {
std::mutex g_tl_mu;
uint64_t* g_tl_buf = nullptr;
int64_t g_tl_waves = 0;
}  // namespace

void set_timeline(uint64_t* buf, int64_t waves) {
    std::lock_guard<std::mutex> lock(g_tl_mu);
    g_tl_buf = waves > 0 ? buf : nullptr;
    g_tl_waves = g_tl_buf ? waves : 0;
}
#endif

hipError_t launch_matmul(Engine e, const uint8_t* Wq, const uint8_t* Xq,
                         int n_slots, const int32_t* batch_index, int n_live,
                         const Shape& s, const Tiling& t, float* Y,
                         void* workspace, hipStream_t st) {
    MmArgs a;
#ifdef Q8_TIMELINE
    {
        std::lock_guard<std::mutex> lock(g_tl_mu);
        a.tl = g_tl_buf;
        a.tl_waves = g_tl_waves;
    }
#endif
    a.CT = n_slots / kMaxSlots;
    if (a.CT < 1 || a.CT * kMaxSlots != n_slots || n_slots > kMaxColumns) return hipErrorInvalidValue;
    a.wq = Wq;
    a.wd = reinterpret_cast<const uint16_t*>(Wq + s.q_bytes);
    a.xq = Xq;
    a.xd = reinterpret_cast<const uint16_t*>(Xq + a.CT * s.act_q_bytes);
    a.xq_gs = s.act_q_bytes;
    a.xd_gs = s.NSC * 4 * (kChunkDBytes / 2);
    a.bidx = batch_index;
    a.Y = Y;
    a.N = s.N;
    a.G = s.G;
    a.KB = (int)s.KB;
    a.NSC = (int)s.NSC;
    a.n_live = n_live;
    a.S = t.splits;
    a.KW = t.kw;
    a.y_vec4 = (s.N % 4 == 0 && reinterpret_cast<uintptr_t>(Y) % 16 == 0) ? 1 : 0;
    if (a.S * a.KW > a.NSC) return hipErrorInvalidValue;
    a.n_whole = 0;
    if (e == Engine::kDot4) return a.CT == 1 ? launch_dot4(a, st) : hipErrorInvalidValue;
    MmPlan p;
    if (!plan_matmul(s, t, n_slots, workspace != nullptr, p)) return hipErrorInvalidValue;
    a.n_rb = p.n_rb;
    a.n_whole = p.n_whole;
    a.recs = p.split ? static_cast<uint8_t*>(workspace) : nullptr;
    if (p.ct == 1) return launch_ct1<false>(a, p.rg, p.split, p.ring, t.nt_weights, st);
    if (p.rg == 1) {
        switch (p.ct) {
            case 2: return launch_mfma<1, 2, 2, true, false>(a, st);
            case 3: return launch_mfma<1, 3, 2, true, false>(a, st);
            case 4: return launch_mfma<1, 4, 2, true, false>(a, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (p.ct) {
        case 2:
            return p.ring == 4 ? launch_mfma<2, 2, 4, true, false>(a, st)
                 : p.ring == 2 ? launch_mfma<2, 2, 2, true, false>(a, st)
                               : launch_mfma<2, 2, 1, true, false>(a, st);
        case 3: return launch_mfma<2, 3, 2, true, false>(a, st);
        case 4:
            return p.ring == 4 ? launch_mfma<2, 4, 4, true, false>(a, st)
                               : launch_mfma<2, 4, 2, true, false>(a, st);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_matmul_fused(const uint8_t* Wq, const float* X, int n_rows,
                               uint8_t* Xq, const int32_t* batch_index, int n_live,
                               const Shape& s, const Tiling& t, float* Y,
                               void* workspace, int max_spins, bool quantize,
                               hipStream_t st) {
    MmArgs a;
#ifdef Q8_TIMELINE
    {  // the matmul workgroups' waves (wave index from the first matmul workgroup)
        std::lock_guard<std::mutex> lock(g_tl_mu);
        a.tl = g_tl_buf;
        a.tl_waves = g_tl_waves;
    }
#endif
    a.CT = 1;
    a.wq = Wq;
    a.wd = reinterpret_cast<const uint16_t*>(Wq + s.q_bytes);
    a.xq = Xq;
    a.xd = reinterpret_cast<const uint16_t*>(Xq + s.act_q_bytes);
    a.xq_gs = s.act_q_bytes;
    a.xd_gs = s.NSC * 4 * (kChunkDBytes / 2);
    a.bidx = batch_index;
    a.Y = Y;
    a.N = s.N;
    a.G = s.G;
    a.KB = (int)s.KB;
    a.NSC = (int)s.NSC;
    a.n_live = n_live;
    a.S = t.splits;
    a.KW = t.kw;
    a.y_vec4 = (s.N % 4 == 0 && reinterpret_cast<uintptr_t>(Y) % 16 == 0) ? 1 : 0;
    a.X = X;
    a.n_rows = n_rows;
    a.max_spins = max_spins;
    a.P = quantize ? -1 : 0;  // -1: as many producers as the slots need
    // page 0 of the workspace: the two top counters and the timeout word,
    // each in its own 128-byte line, then the two sets of sub-counters;
    // pages 1 .. kReadyCopies: the flags
    uint32_t* w32 = static_cast<uint32_t*>(workspace);
    a.qflag = w32;
    a.qexit = w32 + 32;
    a.timeouts = w32 + kFusedTimeoutsOffset / 4;
    a.qflag_sub = w32 + 96;
    a.qexit_sub = a.qflag_sub + kSubCounters * kSubStride;
    a.qready = w32 + kReadyStride;
    static_assert(kFusedTimeoutsOffset == 64 * 4, "timeout word: its own line in page 0");
    static_assert(96 + 2 * kSubCounters * kSubStride <= kReadyStride, "counters fit page 0");
    static_assert((1 + kReadyCopies) * kReadyStride * 4 <= kFusedFlagBytes, "flag pages");
    if (a.S * a.KW > a.NSC) return hipErrorInvalidValue;
    const bool split = t.splits > 1;
    const int rg = launch_rg(s, t, split);
    a.n_rb = (int)((s.G + rg - 1) / rg);
    a.recs = split ? static_cast<uint8_t*>(workspace) + kFusedFlagBytes : nullptr;
    if (t.split_from % rg != 0) return hipErrorInvalidValue;
    a.n_whole = (int)(t.split_from / rg);
    // 4 chunks in flight whatever the tiling says: the weights a wave puts in
    // flight before it waits for the slots are what hides that wait (the
    // ring depth does not change the sums)
    return launch_ct1<true>(a, rg, split, 4, true, st);
}

}  // namespace q8
