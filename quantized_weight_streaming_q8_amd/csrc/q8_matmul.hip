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
// significands).  Each wave owns a contiguous K-slice (a run of 256-value
// super-chunks) and accumulates its terms in ascending block order; the
// KS waves of a workgroup then add their partial sums in wave order through
// LDS.  KS and the slices depend only on (N, K), so the arithmetic of an
// output never depends on n_live or on other tokens.
//
// Two int8 dot engines compute S, with the same accumulation order, so their
// results are bit-identical:
//   * MFMA: one v_mfma_i32_16x16x32_i8 per (16 rows, block) dots the block
//     against 16 token slots at once.  A = activations (token = lane & 15),
//     B = weights (row = lane & 15), D[token][row] -> lane holds row
//     lane & 15 for tokens 4*(lane >> 4) + r.  The cost is the same for any
//     n_live, so the weight stream is the only thing that scales.
//   * DOT4: one output row per lane, v_dot4 over the row's 32 bytes against
//     the token's block (wave-uniform, so it comes through scalar loads).  Its
//     VALU work grows with n_live.
//
// Token slots come from batch_index through the activation slot buffer (the
// batch_index gather of "[feature] Enable Dynamic Batching", section
// "Objective").  Lanes of tokens t >= n_live read token 0's slot and their
// results are dropped; a slot index outside [0,16) is never read through
// (slot 0 is read instead) and its output row is written as NaN.

#include "q8_internal.h"

#include <math.h>

namespace q8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kMaxKs = 16;  // waves per workgroup at most (1024 threads)

__device__ inline uint4 ld16(const void* p) {
    return *reinterpret_cast<const uint4*>(p);
}

// The activation slot buffer is never written while a matmul runs, so a
// wave-uniform address into it may be read through the scalar cache.
typedef __attribute__((address_space(4))) const uint32_t cu32;
typedef __attribute__((address_space(4))) const _Float16 chalf;

__device__ inline float half_at(const uint4& v, int i) {
    const uint32_t w = (i >> 1) == 0 ? v.x : (i >> 1) == 1 ? v.y : (i >> 1) == 2 ? v.z : v.w;
    const uint16_t h = (uint16_t)(w >> (16 * (i & 1)));
    return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline int live_slot(const int32_t* __restrict__ bidx, int n_live, int t) {
    const int s = bidx[t < n_live ? t : 0];
    return (s >= 0 && s < kMaxSlots) ? s : 0;
}

__device__ inline bool slot_bad(const int32_t* __restrict__ bidx, int t) {
    const int s = bidx[t];
    return s < 0 || s >= kMaxSlots;
}

__device__ inline float term_fma(int S, float dwf, float dxf, float acc) {
    const float p = __builtin_fmaf(dwf, dxf, 0.0f);  // exact product
    return __builtin_fmaf((float)S, p, acc);
}

// ------------------------------------------------------------------------
// MFMA engine
// ------------------------------------------------------------------------

struct MfmaArgs {
    const uint8_t* wq;     // packed q region
    const uint16_t* wd;    // packed scale region
    const uint8_t* xq;     // activation slot buffer
    const int32_t* bidx;   // batch_index
    float* Y;
    int64_t N;
    int64_t G;
    int64_t stride;        // activation slot stride
    int64_t Kp;
    int KB, NSC, KS, n_live;
};

// One super-chunk (8 blocks) for RG row groups.
template <int RG, bool TAIL>
__device__ inline void mfma_step(int sc, int nb, const uint8_t* xa,
                                 const uint16_t* const xd[4],
                                 const uint8_t* const wrow[RG],
                                 const uint16_t* const wdrow[RG],
                                 float acc[RG][4]) {
    uint4 aq[4], ad[4], wv[RG][4], wdv[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
#pragma unroll
        for (int c = 0; c < 4; ++c) wv[rg][c] = ld16(wrow[rg] + (int64_t)sc * kScQBytes + c * kChunkBytes);
        wdv[rg] = ld16(wdrow[rg] + (int64_t)sc * (kScDBytes / 2));
    }
#pragma unroll
    for (int c = 0; c < 4; ++c) aq[c] = ld16(xa + (int64_t)sc * kScValues + c * 64);
#pragma unroll
    for (int r = 0; r < 4; ++r) ad[r] = ld16(xd[r] + sc * kScBlocks);

#pragma unroll
    for (int c = 0; c < 4; ++c) {
        // lanes 0-31 hold block 2c (bytes 16s..16s+15), lanes 32-63 block
        // 2c+1: swap 8 bytes across the halves so every lane holds its k-slot
        // of both blocks.
        const auto s02 = __builtin_amdgcn_permlane32_swap(aq[c].x, aq[c].z, false, false);
        const auto s13 = __builtin_amdgcn_permlane32_swap(aq[c].y, aq[c].w, false, false);
        const long xa0 = (long)((uint64_t)s02[0] | ((uint64_t)s13[0] << 32));
        const long xa1 = (long)((uint64_t)s02[1] | ((uint64_t)s13[1] << 32));
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const long w0 = (long)((uint64_t)wv[rg][c].x | ((uint64_t)wv[rg][c].y << 32));
            const long w1 = (long)((uint64_t)wv[rg][c].z | ((uint64_t)wv[rg][c].w << 32));
            const v4i zero = {0, 0, 0, 0};
            const v4i S0 = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa0, w0, zero, 0, 0, 0);
            const v4i S1 = __builtin_amdgcn_mfma_i32_16x16x32_i8(xa1, w1, zero, 0, 0, 0);
            const int b0 = 2 * c, b1 = 2 * c + 1;
            if (!TAIL || b0 < nb) {
                const float dwf = half_at(wdv[rg], b0);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rg][r] = term_fma(S0[r], dwf, half_at(ad[r], b0), acc[rg][r]);
            }
            if (!TAIL || b1 < nb) {
                const float dwf = half_at(wdv[rg], b1);
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[rg][r] = term_fma(S1[r], dwf, half_at(ad[r], b1), acc[rg][r]);
            }
        }
    }
}

template <int RG>
__global__ void __launch_bounds__(1024)
mm_mfma_kernel(MfmaArgs a) {
    extern __shared__ float red[];  // [KS][RG][4][64] when KS > 1
    const int lane = threadIdx.x & 63;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int64_t g0 = (int64_t)blockIdx.x * RG;
    const int sc0 = (int)(((int64_t)ks * a.NSC) / a.KS);
    const int sc1 = (int)(((int64_t)(ks + 1) * a.NSC) / a.KS);

    // activation operand: token lane & 15, 16 bytes at 64c + 16*(lane >> 4)
    const int sa = live_slot(a.bidx, a.n_live, lane & 15);
    const uint8_t* xa = a.xq + (int64_t)sa * a.stride + 16 * (lane >> 4);
    const uint16_t* xd[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int s = live_slot(a.bidx, a.n_live, 4 * (lane >> 4) + r);
        xd[r] = reinterpret_cast<const uint16_t*>(a.xq + (int64_t)s * a.stride + a.Kp);
    }
    const uint8_t* wrow[RG];
    const uint16_t* wdrow[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int64_t g = min(g0 + rg, a.G - 1);  // past-the-end groups redo the last one
        wrow[rg] = a.wq + g * a.NSC * kScQBytes + lane * 16;
        wdrow[rg] = a.wd + g * a.NSC * (kScDBytes / 2) + (lane & 15) * 8;
    }

    float acc[RG][4];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[rg][r] = 0.0f;

    const int sc_full = min(sc1, a.KB / kScBlocks);
    int sc = sc0;
    for (; sc < sc_full; ++sc) mfma_step<RG, false>(sc, kScBlocks, xa, xd, wrow, wdrow, acc);
    if (sc < sc1) mfma_step<RG, true>(sc, a.KB - sc * kScBlocks, xa, xd, wrow, wdrow, acc);

    if (a.KS == 1) {
#pragma unroll
        for (int rg = 0; rg < RG; ++rg)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * (lane >> 4) + r;
                const int64_t n = (g0 + rg) * kRowsPerGroup + (lane & 15);
                if (t < a.n_live && n < a.N)
                    a.Y[(int64_t)t * a.N + n] = slot_bad(a.bidx, t) ? __builtin_nanf("") : acc[rg][r];
            }
        return;
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[((ks * RG + rg) * 4 + r) * 64 + lane] = acc[rg][r];
    __syncthreads();
    for (int e = threadIdx.x; e < RG * 256; e += a.KS * 64) {
        float y = red[e];
        for (int k = 1; k < a.KS; ++k) y += red[k * RG * 256 + e];
        const int rg = e >> 8, r = (e >> 6) & 3, ln = e & 63;
        const int t = 4 * (ln >> 4) + r;
        const int64_t n = (g0 + rg) * kRowsPerGroup + (ln & 15);
        if (t < a.n_live && n < a.N)
            a.Y[(int64_t)t * a.N + n] = slot_bad(a.bidx, t) ? __builtin_nanf("") : y;
    }
}

// ------------------------------------------------------------------------
// DOT4 engine: one row per lane, 64 rows (4 row groups) per wave.
// ------------------------------------------------------------------------

template <int NT, bool TAIL>
__device__ inline void dot4_step(int sc, int nb, const uint8_t* wrow,
                                 const uint16_t* wdrow,
                                 const uint8_t* const xrow[NT], int64_t Kp,
                                 float acc[NT]) {
    const uint4 wdv = ld16(wdrow + (int64_t)sc * (kScDBytes / 2));
    // token scales of the 8 blocks: 4 dwords of two halves each, scalar loads
    uint32_t dxw[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        cu32* dp = (cu32*)(xrow[t] + Kp + (int64_t)sc * kScBlocks * 2);
#pragma unroll
        for (int i = 0; i < 4; ++i) dxw[t][i] = dp[i];
    }
#pragma unroll 1
    for (int c = 0; c < 4; ++c) {
        if (TAIL && 2 * c >= nb) break;
        uint4 w[4];  // [k-slot]: this row's 8 bytes of blocks 2c and 2c+1
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] = ld16(wrow + (int64_t)sc * kScQBytes + c * kChunkBytes + s * 256);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int bb = 2 * c + h;
            if (TAIL && bb >= nb) continue;
            const int64_t b = (int64_t)sc * kScBlocks + bb;
            const float dwf = half_at(wdv, bb);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                cu32* ap = (cu32*)(xrow[t] + b * kBlock);
                int S = 0;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int p4 = slot_pos(s) / 4;
                    const uint32_t wlo = h ? w[s].z : w[s].x;
                    const uint32_t whi = h ? w[s].w : w[s].y;
                    S = __builtin_amdgcn_sdot4((int)wlo, (int)ap[p4], S, false);
                    S = __builtin_amdgcn_sdot4((int)whi, (int)ap[p4 + 1], S, false);
                }
                // dxw[t][c] holds the halves of blocks 2c (low) and 2c+1 (high)
                uint32_t dsel = dxw[t][0];
#pragma unroll
                for (int i = 1; i < 4; ++i) dsel = (c == i) ? dxw[t][i] : dsel;
                const uint16_t dh = (uint16_t)(dsel >> (16 * h));
                acc[t] = term_fma(S, dwf, (float)__builtin_bit_cast(_Float16, dh), acc[t]);
            }
        }
    }
}

template <int NT>
__global__ void __launch_bounds__(1024)
mm_dot4_kernel(MfmaArgs a) {
    extern __shared__ float red[];  // [KS][NT][64] when KS > 1
    const int lane = threadIdx.x & 63;
    const int ks = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
    const int64_t g0 = (int64_t)blockIdx.x * 4;
    const int sc0 = (int)(((int64_t)ks * a.NSC) / a.KS);
    const int sc1 = (int)(((int64_t)(ks + 1) * a.NSC) / a.KS);
    const int64_t g = min(g0 + (lane >> 4), a.G - 1);
    const int j = lane & 15;
    const uint8_t* wrow = a.wq + g * a.NSC * kScQBytes + j * 16;
    const uint16_t* wdrow = a.wd + g * a.NSC * (kScDBytes / 2) + j * 8;
    const uint8_t* xrow[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int s = __builtin_amdgcn_readfirstlane(live_slot(a.bidx, a.n_live, t));
        xrow[t] = a.xq + (int64_t)s * a.stride;
    }
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.0f;

    const int sc_full = min(sc1, a.KB / kScBlocks);
    int sc = sc0;
    for (; sc < sc_full; ++sc) dot4_step<NT, false>(sc, kScBlocks, wrow, wdrow, xrow, a.Kp, acc);
    if (sc < sc1) dot4_step<NT, true>(sc, a.KB - sc * kScBlocks, wrow, wdrow, xrow, a.Kp, acc);

    const int64_t n = (g0 + (lane >> 4)) * kRowsPerGroup + j;
    if (a.KS == 1) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            if (n < a.N) a.Y[(int64_t)t * a.N + n] = slot_bad(a.bidx, t) ? __builtin_nanf("") : acc[t];
        return;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) red[(ks * NT + t) * 64 + lane] = acc[t];
    __syncthreads();
    for (int e = threadIdx.x; e < NT * 64; e += a.KS * 64) {
        float y = red[e];
        for (int k = 1; k < a.KS; ++k) y += red[k * NT * 64 + e];
        const int t = e >> 6, ln = e & 63;
        const int64_t nn = (g0 + (ln >> 4)) * kRowsPerGroup + (ln & 15);
        if (nn < a.N) a.Y[(int64_t)t * a.N + nn] = slot_bad(a.bidx, t) ? __builtin_nanf("") : y;
    }
}

template <int NT>
hipError_t launch_dot4_nt(const MfmaArgs& a, hipStream_t st) {
    const unsigned grid = (unsigned)((a.G + 3) / 4);
    const size_t lds = a.KS > 1 ? (size_t)a.KS * NT * 64 * sizeof(float) : 0;
    hipLaunchKernelGGL(mm_dot4_kernel<NT>, dim3(grid), dim3(64 * a.KS), lds, st, a);
    return hipGetLastError();
}

hipError_t launch_dot4(const MfmaArgs& a, hipStream_t st) {
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

Tiling choose_tiling(const Shape& s) {
    // Enough waves to keep ~4096 weight streams in flight across 256 CUs,
    // never more K-slices than super-chunks or than a workgroup can hold.
    Tiling t;
    int64_t ks = (4096 + s.G - 1) / s.G;
    ks = std::min<int64_t>(ks, std::min<int64_t>(kMaxKs, s.NSC));
    t.ks = (int)std::max<int64_t>(ks, 1);
    return t;
}

hipError_t launch_matmul(Engine e, const uint8_t* Wq, const uint8_t* Xq,
                         const int32_t* batch_index, int n_live,
                         const Shape& s, const Tiling& t, float* Y,
                         hipStream_t st) {
    MfmaArgs a;
    a.wq = Wq;
    a.wd = reinterpret_cast<const uint16_t*>(Wq + s.q_bytes);
    a.xq = Xq;
    a.bidx = batch_index;
    a.Y = Y;
    a.N = s.N;
    a.G = s.G;
    a.stride = s.stride;
    a.Kp = s.Kp;
    a.KB = (int)s.KB;
    a.NSC = (int)s.NSC;
    a.KS = t.ks;
    a.n_live = n_live;
    if (e == Engine::kDot4) return launch_dot4(a, st);
    constexpr int RG = 1;
    const unsigned grid = (unsigned)((s.G + RG - 1) / RG);
    const size_t lds = t.ks > 1 ? (size_t)t.ks * RG * 256 * sizeof(float) : 0;
    hipLaunchKernelGGL(mm_mfma_kernel<RG>, dim3(grid), dim3(64 * t.ks), lds, st, a);
    return hipGetLastError();
}

}  // namespace q8
