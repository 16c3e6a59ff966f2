// q8_rope.hip -- pos-vector rotary position embedding for gfx950.
//
// "Batched decode: co-decode N live sessions in one GPU pass" (antirez/ds4
// PR #530), commit "CUDA: add pos-vector RoPE tail variants": in a batched
// decode step every row (token) sits at its own position, so the rotation
// reads a small per-row position array, and each row must come out bitwise
// as a single-row launch would make it.  Here every output depends only on
// its own row's two inputs and position, through the same instructions, so
// a row's bits never depend on the other rows.
//
// The rotation is the plain rotary embedding with the rotate-half pairing:
// in each head of head_dim values, values i and i + head_dim/2 turn by
// theta = pos * base^(-2i/head_dim).  The angle, its sine and cosine and the
// rotation are evaluated in double (so positions far into a long context
// keep their accuracy) and each result is rounded once to fp32.
//
// One thread per pair, in place; the pairs of a row are contiguous in i, so
// a wave reads and writes contiguous runs of a row.

#include "q8_internal.h"

#include <math.h>

namespace q8 {
namespace {

constexpr int kRopeThreads = 256;

__global__ void __launch_bounds__(kRopeThreads)
rope_multi_kernel(float* __restrict__ Y, int64_t row_stride, const int32_t* __restrict__ pos,
                  int n_heads, int half, double neg_two_over_d, double log2_base, int64_t total) {
    const int64_t tid = (int64_t)blockIdx.x * kRopeThreads + threadIdx.x;
    if (tid >= total) return;
    const int i = (int)(tid % half);
    const int64_t th = tid / half;
    const int h = (int)(th % n_heads);
    const int64_t t = th / n_heads;
    // base^(-2i/d) = exp2(log2(base) * (-2i/d)), in double
    const double inv_freq = exp2(log2_base * ((double)i * neg_two_over_d));
    const double theta = (double)pos[t] * inv_freq;
    double s, c;
    sincos(theta, &s, &c);
    float* p = Y + t * row_stride + (int64_t)h * 2 * half + i;
    const double a = p[0], b = p[half];
    p[0] = (float)(a * c - b * s);
    p[half] = (float)(a * s + b * c);
}

}  // namespace

hipError_t launch_rope_multi(float* Y, int n_rows, int64_t row_stride, const int32_t* pos,
                             int n_heads, int head_dim, double base, hipStream_t st) {
    const int half = head_dim / 2;
    const int64_t total = (int64_t)n_rows * n_heads * half;
    const unsigned grid = (unsigned)((total + kRopeThreads - 1) / kRopeThreads);
    hipLaunchKernelGGL(rope_multi_kernel, dim3(grid), dim3(kRopeThreads), 0, st, Y, row_stride,
                       pos, n_heads, half, -2.0 / (double)head_dim, log2(base), total);
    return hipGetLastError();
}

}  // namespace q8
