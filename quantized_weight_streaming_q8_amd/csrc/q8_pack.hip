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
// Thread mapping, all kernels: one lane per 8-value segment, 4 consecutive
// lanes per 32-value block, consecutive blocks of a row on consecutive lane
// groups, so a wave reads 2 KB of contiguous fp32 per row.

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

__global__ void __launch_bounds__(kThreads)
pack_weights_kernel(const float* __restrict__ W, int64_t N, int64_t K,
                    int64_t KB, int64_t NSC, int64_t total,
                    uint8_t* __restrict__ wq, uint16_t* __restrict__ wd) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= total) return;  // total is a multiple of 4: groups exit whole
    const SegIndex ix = seg_index(tid, NSC * kScBlocks);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ix.row < N && ix.blk < KB) load8(W + ix.row * K + ix.blk * kBlock + ix.seg * 8, v);
    const QuantSeg r = quantize_segment(v);
    *reinterpret_cast<uint2*>(wq + packed_q_offset(ix.row, ix.blk, ix.seg, NSC)) =
        make_uint2(r.lo, r.hi);
    if (ix.seg == 0) wd[packed_d_index(ix.row, ix.blk, NSC)] = r.d16;
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
// rows < n_rows are written.
__global__ void __launch_bounds__(kThreads)
quantize_acts_kernel(const float* __restrict__ X, int64_t K, int64_t KB,
                     int64_t NSC, int64_t total, uint8_t* __restrict__ xq,
                     uint16_t* __restrict__ xd) {
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (tid >= total) return;
    const SegIndex ix = seg_index(tid, NSC * kScBlocks);
    float v[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (ix.blk < KB) load8(X + ix.row * K + ix.blk * kBlock + ix.seg * 8, v);
    const QuantSeg r = quantize_segment(v);
    *reinterpret_cast<uint2*>(xq + packed_q_offset(ix.row, ix.blk, ix.seg, NSC)) =
        make_uint2(r.lo, r.hi);
    if (ix.seg == 0) xd[packed_d_index(ix.row, ix.blk, NSC)] = r.d16;
}

inline unsigned grid_for(int64_t total) {
    return (unsigned)((total + kThreads - 1) / kThreads);
}

}  // namespace

hipError_t launch_pack_weights(const float* W, const Shape& s, uint8_t* Wq,
                               hipStream_t st) {
    const int64_t total = s.G * kRowsPerGroup * s.NSC * kScBlocks * 4;
    uint16_t* wd = reinterpret_cast<uint16_t*>(Wq + s.q_bytes);
    hipLaunchKernelGGL(pack_weights_kernel, dim3(grid_for(total)), dim3(kThreads),
                       0, st, W, s.N, s.K, s.KB, s.NSC, total, Wq, wd);
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
    const int64_t total = (int64_t)n_rows * s.NSC * kScBlocks * 4;
    uint16_t* xd = reinterpret_cast<uint16_t*>(Xq + (n_slots / kMaxSlots) * s.act_q_bytes);
    hipLaunchKernelGGL(quantize_acts_kernel, dim3(grid_for(total)), dim3(kThreads),
                       0, st, X, s.K, s.KB, s.NSC, total, Xq, xd);
    return hipGetLastError();
}

}  // namespace q8
