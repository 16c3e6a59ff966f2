// q8_pack.hip -- q8_0 weight packer, import/export of canonical q8_0, and the
// activation pre-quantiser.
//
// Quantisation follows the q8_0 block of "Batched decode: co-decode N live
// sessions in one GPU pass" (antirez/ds4 PR #530), section "Why it's worth it
// -- the narrow-batch matmul" (32-weight blocks, pre-quantised activations),
// read as the GGUF q8_0 block: d = absmax/127 in binary32, q = round half away
// from zero of x/d (IEEE division), clamped to +-127, d stored as binary16.
// An activation slot buffer of n_slots slots uses the packed layout of an
// n_slots-row matrix (row = slot).
//
// Thread mapping.  The weight packer: one wave per chunk of the packed
// layout (16 rows x 2 blocks, 1 KB), lane l holding exactly the 16 bytes it
// stores at l*16: row l & 15, k-slot l >> 4, 8 values of each of the two
// blocks.  Every wave's q store is one contiguous 1 KB and its scale store
// 64 contiguous bytes; a block's 4 segments sit in lanes 16 apart.  Import
// and export: one lane per 8-value segment, 4 consecutive lanes per block,
// consecutive blocks of a row on consecutive lane groups.  The activation
// pre-quantiser: the same order with 2 or 4 values per lane (16 or 8 lanes
// per block), and one-wave workgroups, which spread the few waves of the
// 16 short slot rows over the most CUs.

#include "q8_internal.h"

namespace q8 {
namespace {

constexpr int kThreads = 256;

struct SegIndex {
    int64_t row;  // row (weights: 0..16G-1, activations: 0..n_rows-1)
    int64_t blk;  // block within the padded row, 0..8*NSC-1
    int seg;      // 8-value segment within the block, 0..3
};

__device__ inline SegIndex seg_index(int64_t tid, int64_t blocks_per_row) {
    SegIndex ix;
    ix.seg = (int)(tid & 3);
    const int64_t b = tid >> 2;
    ix.blk = b % blocks_per_row;
    ix.row = b / blocks_per_row;
    return ix;
}

__device__ inline void load8(const float* p, float v[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Quantise rows [16g, 16g+16) x blocks [2cg, 2cg+2) of the row-major fp32
// W (N x K) into chunk cg of row group g of the packed layout.  Rows past N
// and blocks past K are written as zeros, the layout's padding.
__global__ void __launch_bounds__(kThreads)
pack_weights_kernel(const float* __restrict__ W, int64_t N, int64_t K, int64_t KB,
                    int64_t NSC, int64_t n_waves, uint8_t* __restrict__ wq,
                    uint16_t* __restrict__ wd) {
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wave >= n_waves) return;  // wave-uniform
    const int lane = threadIdx.x & 63;
    const int64_t chunks = NSC * 4;
    const int64_t g = wave / chunks, cg = wave % chunks;
    const int64_t row = g * kRowsPerGroup + (lane & 15);
    const int ks = lane >> 4;
    uint32_t out[4];
    uint32_t dd = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t blk = 2 * cg + h;
        float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (row < N && blk < KB) load8(W + row * K + blk * kBlock + slot_pos(ks), v);
        const QuantSeg r = quantize_segment<16>(v);
        out[2 * h] = r.lo;
        out[2 * h + 1] = r.hi;
        dd |= (uint32_t)r.d16 << (16 * h);
    }
    *reinterpret_cast<uint4*>(wq + (g * chunks + cg) * kChunkBytes + lane * 16) =
        make_uint4(out[0], out[1], out[2], out[3]);
    if (ks == 0)  // blocks 2cg and 2cg+1 of this row: scale halves 2j, 2j+1 of the chunk
        *reinterpret_cast<uint32_t*>(wd + ((g * chunks + cg) * kRowsPerGroup + (lane & 15)) * 2) = dd;
}

__global__ void __launch_bounds__(kThreads)
pack_weights_q_kernel(const int8_t* __restrict__ q, const uint16_t* __restrict__ d16,
                      int64_t N, int64_t K, int64_t KB, int64_t NSC,
                      int64_t total, uint8_t* __restrict__ wq,
                      uint16_t* __restrict__ wd) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= total) return;
    const SegIndex ix = seg_index(tid, NSC * kScBlocks);
    uint2 v = make_uint2(0u, 0u);
    uint16_t d = 0;
    if (ix.row < N && ix.blk < KB) {
        v = *reinterpret_cast<const uint2*>(q + ix.row * K + ix.blk * kBlock + ix.seg * 8);
        d = d16[ix.row * KB + ix.blk];
    }
    *reinterpret_cast<uint2*>(wq + packed_q_offset(ix.row, ix.blk, ix.seg, NSC)) = v;
    if (ix.seg == 0) wd[packed_d_index(ix.row, ix.blk, NSC)] = d;
}

__global__ void __launch_bounds__(kThreads)
unpack_weights_kernel(const uint8_t* __restrict__ wq, const uint16_t* __restrict__ wd,
                      int64_t N, int64_t K, int64_t KB, int64_t NSC,
                      int64_t total, int8_t* __restrict__ q,
                      uint16_t* __restrict__ d16) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= total) return;
    const SegIndex ix = seg_index(tid, KB);  // canonical blocks only
    *reinterpret_cast<uint2*>(q + ix.row * K + ix.blk * kBlock + ix.seg * 8) =
        *reinterpret_cast<const uint2*>(wq + packed_q_offset(ix.row, ix.blk, ix.seg, NSC));
    if (ix.seg == 0) d16[ix.row * KB + ix.blk] = wd[packed_d_index(ix.row, ix.blk, NSC)];
}

// Activations go to the packed layout of an n_slots-row matrix (row = slot); only
// rows < n_rows are written.  A block is quantised by 32 / E consecutive
// lanes, E consecutive values each: the short 16-row input then spreads over
// many waves, each with few serial divisions, which is what the kernel's
// latency depends on.  total = n_rows x 8 NSC x 32 / E (whole lane groups).
template <int E>
__global__ void __launch_bounds__(64)
quantize_acts_kernel(const float* __restrict__ X, int64_t K, int64_t KB,
                     int64_t NSC, int64_t total, uint8_t* __restrict__ xq,
                     uint16_t* __restrict__ xd) {
    constexpr int G = 32 / E;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (tid >= total) return;  // whole groups of G lanes: G divides 64 and total
    const int part = (int)(tid % G);
    const int64_t b = tid / G;
    const int64_t blk = b % (NSC * kScBlocks), row = b / (NSC * kScBlocks);
    float v[E];
#pragma unroll
    for (int i = 0; i < E; ++i) v[i] = 0.0f;
    if (blk < KB) {
        const float* p = X + row * K + blk * kBlock + part * E;
        if constexpr (E == 2) {
            const float2 a = *reinterpret_cast<const float2*>(p);
            v[0] = a.x; v[1] = a.y;
        } else if constexpr (E == 4) {
            const float4 a = *reinterpret_cast<const float4*>(p);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        } else {
            load8(p, v);
        }
    }
    uint32_t q[(E + 3) / 4];
    const uint16_t d16 = quantize_values<E>(v, q);
    // values part*E .. part*E + E - 1 of the block: segment (part*E) / 8, from
    // byte (part*E) % 8 of it
    uint8_t* dst = xq + packed_q_offset(row, blk, (part * E) >> 3, NSC) + ((part * E) & 7);
    if constexpr (E == 2) *reinterpret_cast<uint16_t*>(dst) = (uint16_t)q[0];
    else if constexpr (E == 4) *reinterpret_cast<uint32_t*>(dst) = q[0];
    else *reinterpret_cast<uint2*>(dst) = make_uint2(q[0], q[1]);
    if (part == 0) xd[packed_d_index(row, blk, NSC)] = d16;
}

inline unsigned grid_for(int64_t total) {
    return (unsigned)((total + kThreads - 1) / kThreads);
}

}  // namespace

hipError_t launch_pack_weights(const float* W, const Shape& s, uint8_t* Wq,
                               hipStream_t st) {
    const int64_t waves = s.G * s.NSC * 4;  // one per chunk
    uint16_t* wd = reinterpret_cast<uint16_t*>(Wq + s.q_bytes);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(waves * 64)), dim3(kThreads),
                       0, st, W, s.N, s.K, s.KB, s.NSC, waves, Wq, wd);
    return hipGetLastError();
}

hipError_t launch_pack_weights_q(const int8_t* q, const uint16_t* d16,
                                 const Shape& s, uint8_t* Wq, hipStream_t st) {
    const int64_t total = s.G * kRowsPerGroup * s.NSC * kScBlocks * 4;
    uint16_t* wd = reinterpret_cast<uint16_t*>(Wq + s.q_bytes);
    hipLaunchKernelGGL(pack_weights_q_kernel, dim3(grid_for(total)), dim3(kThreads),
                       0, st, q, d16, s.N, s.K, s.KB, s.NSC, total, Wq, wd);
    return hipGetLastError();
}

hipError_t launch_unpack_weights(const uint8_t* Wq, const Shape& s, int8_t* q,
                                 uint16_t* d16, hipStream_t st) {
    const int64_t total = s.N * s.KB * 4;
    const uint16_t* wd = reinterpret_cast<const uint16_t*>(Wq + s.q_bytes);
    hipLaunchKernelGGL(unpack_weights_kernel, dim3(grid_for(total)), dim3(kThreads),
                       0, st, Wq, wd, s.N, s.K, s.KB, s.NSC, total, q, d16);
    return hipGetLastError();
}

hipError_t launch_quantize_acts(const float* X, int n_rows, const Shape& s,
                                uint8_t* Xq, int n_slots, hipStream_t st) {
    uint16_t* xd = reinterpret_cast<uint16_t*>(Xq + (n_slots / kMaxSlots) * s.act_q_bytes);
    const int64_t blocks = (int64_t)n_rows * s.NSC * kScBlocks;
    // measured in graph replays (one launch is ~2.1-2.5 us, most of it the
    // launch itself): 2 values per lane up to about 1000 waves (16 rows of
    // K <= 8192: 2.10 against 2.18 us with 4 and 2.31 with 8 at K = 5120),
    // 4 above (16 x 17408: 2.47 against 2.64 with 2 and 2.51 with 8)
    if (blocks * 16 <= (int64_t)16 * 8192 / 2) {
        const int64_t total = blocks * 16;
        hipLaunchKernelGGL(quantize_acts_kernel<2>, dim3((unsigned)((total + 63) / 64)), dim3(64), 0,
                           st, X, s.K, s.KB, s.NSC, total, Xq, xd);
    } else {
        const int64_t total = blocks * 8;
        hipLaunchKernelGGL(quantize_acts_kernel<4>, dim3((unsigned)((total + 63) / 64)), dim3(64), 0,
                           st, X, s.K, s.KB, s.NSC, total, Xq, xd);
    }
    return hipGetLastError();
}

}  // namespace q8
