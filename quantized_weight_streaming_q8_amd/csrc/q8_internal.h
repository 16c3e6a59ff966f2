// q8_internal.h -- layouts and launch helpers shared by the q8narrow kernels.
//
// Packed weight layout (private).  The matrix is cut into row groups of 16
// rows (the N side of one v_mfma_i32_16x16x32_i8) and, along K, into
// super-chunks of 8 q8_0 blocks (256 values); a super-chunk is 4 chunks of 2
// blocks.  G = ceil(N/16) row groups, NSC = ceil(K/256) super-chunks; rows and
// blocks past the matrix are zero (q = 0, d = 0).
//
//   q region, 4096 bytes per (group, super-chunk), groups outermost:
//     byte ((g*NSC + sc)*4 + c)*1024 + lane*16 + h*8 + e
//       = q[row 16g + (lane & 15)][k = 32*(8sc + 2c + h) + P(lane >> 4) + e]
//     with P = {0, 16, 8, 24}.  One 16-byte load per lane of a wave64 then
//     holds this lane's 8-byte B operand of the MFMA for block 2c (h = 0) and
//     block 2c+1 (h = 1): row = lane & 15, k-slot = lane >> 4.
//   scale region, after the q region, 64 bytes per (group, chunk):
//     half ((g*4*NSC + c)*16 + j)*2 + h = d[row 16g + j][block 2c + h]
//     (c = chunk index along the row).  Four consecutive rows' scales of a
//     chunk are 16 contiguous bytes, the operand of one lane of the MFMA
//     output (rows 4*(lane >> 4) .. +3).
//
// The same layout holds the activation slot buffer: it is the packed form of a
// 16 x K matrix whose row s is slot s.  A lane (token t = lane & 15, k-slot
// g = lane >> 4) of the MFMA engine then finds its 8-byte A operand for blocks
// 2c and 2c+1 in one 16-byte load at chunk offset (g*16 + slot)*16, and a
// wave's activation load for one chunk of all 16 slots is 1 KB contiguous.
// P is the k-slot -> byte-in-block map both operands share; any permutation
// is exact, since a block's 32 products are summed in integers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q8 {

constexpr int kBlock = 32;        // values per q8_0 block
constexpr int kMaxSlots = 16;     // activation slots
constexpr int kMaxColumns = 64;   // slots of a multi-column buffer
constexpr int kRowsPerGroup = 16; // rows per row group
constexpr int kScBlocks = 8;      // blocks per super-chunk
constexpr int kScValues = kScBlocks * kBlock;            // 256
constexpr int kScQBytes = kRowsPerGroup * kScValues;     // 4096
constexpr int kScDBytes = kRowsPerGroup * kScBlocks * 2; // 256
constexpr int kChunkDBytes = kRowsPerGroup * 2 * 2;       // 64
constexpr int kChunkBytes = 1024;                        // 2 blocks x 16 rows

struct Shape {
    int64_t N, K;
    int64_t KB;   // blocks per row
    int64_t G;    // row groups
    int64_t NSC;  // super-chunks per row
    int64_t Kp;   // K padded to a multiple of 256
    int64_t q_bytes;  // packed q region
    int64_t d_bytes;  // packed scale region
    int64_t act_q_bytes;  // activation buffer: q region per 16 slots
};

inline __host__ __device__ int64_t align_up(int64_t v, int64_t a) {
    return (v + a - 1) / a * a;
}

inline Shape make_shape(int64_t N, int64_t K) {
    Shape s;
    s.N = N;
    s.K = K;
    s.KB = K / kBlock;
    s.G = (N + kRowsPerGroup - 1) / kRowsPerGroup;
    s.NSC = (s.KB + kScBlocks - 1) / kScBlocks;
    s.Kp = s.NSC * kScValues;
    s.q_bytes = s.G * s.NSC * kScQBytes;
    s.d_bytes = s.G * s.NSC * kScDBytes;
    s.act_q_bytes = s.NSC * kScQBytes;
    return s;
}

// k-slot of the MFMA operand -> starting byte inside the 32-value block
__host__ __device__ constexpr int slot_pos(int slot) {
    return 8 * (((slot & 1) << 1) | (slot >> 1));
}
// byte offset inside the block (multiple of 8) -> k-slot (inverse of slot_pos)
__host__ __device__ constexpr int pos_slot(int pos8) {
    return ((pos8 & 1) << 1) | (pos8 >> 1);
}

// Byte offset, inside a packed q region, of the 8-byte piece holding segment
// `seg` (8 values) of block `blk` of row `row`.
__device__ inline int64_t packed_q_offset(int64_t row, int64_t blk, int seg,
                                          int64_t NSC) {
    const int64_t g = row >> 4;
    const int j = (int)(row & 15);
    const int64_t sc = blk >> 3;
    const int bb = (int)(blk & 7);
    const int c = bb >> 1, h = bb & 1;
    const int slot = pos_slot(seg);
    return ((g * NSC + sc) * 4 + c) * kChunkBytes + (slot * 16 + j) * 16 + h * 8;
}

// Index (in halves) of the scale of block `blk` of row `row` in a packed
// scale region: [group][chunk][16 rows][2 blocks].
__device__ inline int64_t packed_d_index(int64_t row, int64_t blk, int64_t NSC) {
    const int64_t g = row >> 4;
    const int j = (int)(row & 15);
    const int64_t c = blk >> 1;
    return ((g * 4 * NSC + c) * 16 + j) * 2 + (blk & 1);
}

// ------------------------------------------------------------------------
// q8_0 quantisation of a 32-value block held by a group of G = 32 / E
// lanes, E consecutive values each: lane p of the group (p = 0 .. G-1) is
// lane l0 + p*L, where l0 is a multiple of G*L (L = 1: G consecutive lanes;
// L = 16: lanes 16 apart).  All of them must be active.  Each lane gets its
// E codes (little-endian bytes of q[]) and the block's binary16 scale.
//
// Blocks the format leaves undefined follow one stated rule each: a block
// holding a NaN or an infinity stores q = 0 and the binary16 quiet NaN
// 0x7E00 (every output that uses it is then NaN); a block whose scale
// absmax/127 rounds to zero (absmax 0, or so small the quotient underflows)
// is the zero block, q = 0 and d = +0.
// ------------------------------------------------------------------------
constexpr uint16_t kNanScale = 0x7E00;  // binary16 quiet NaN

template <int E, int L = 1>
__device__ inline uint16_t quantize_values(const float v[E], uint32_t q[(E + 3) / 4]) {
    static_assert(E == 2 || E == 4 || E == 8, "values per lane");
    static_assert(L == 1 || L == 16, "lane distance of a block's lanes");
    constexpr int G = 32 / E;
#pragma unroll
    for (int i = 0; i < (E + 3) / 4; ++i) q[i] = 0u;
    // absmax, with a NaN or an infinity counted as +infinity (fmaxf alone
    // would drop a NaN)
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i) {
        const float m = fabsf(v[i]);
        a = fmaxf(a, m <= __FLT_MAX__ ? m : __builtin_inff());
    }
    // absmax of the 32-value block across the group (max is exact in any order)
#pragma unroll
    for (int m = 1; m < G; m <<= 1) a = fmaxf(a, __shfl_xor(a, m * L, G * L));
    if (!(a <= __FLT_MAX__)) return kNanScale;  // a NaN or an infinity in the block
    const float d = a / 127.0f;                    // correctly rounded (no fast-math)
    if (d == 0.0f) return 0;                       // the zero block, or a scale that underflows
#pragma unroll
    for (int i = 0; i < E; ++i) {
        float x = roundf(v[i] / d);  // IEEE division, ties away from zero
        x = fminf(fmaxf(x, -127.0f), 127.0f);
        const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)x;
        q[i >> 2] |= b << (8 * (i & 3));
    }
    return __builtin_bit_cast(uint16_t, (_Float16)d);  // round to nearest even
}

// One 8-value segment by a group of 4 lanes (the packer's and the fused
// producers' mapping).
struct QuantSeg {
    uint32_t lo, hi;  // 8 int8 values, little-endian
    uint16_t d16;     // binary16 scale of the block
};

template <int L = 1>
__device__ inline QuantSeg quantize_segment(const float v[8]) {
    uint32_t q[2];
    QuantSeg r;
    r.d16 = quantize_values<8, L>(v, q);
    r.lo = q[0];
    r.hi = q[1];
    return r;
}

// ------------------------------------------------------------------------
// Kernel launchers (host).  Shapes and pointers are validated by the caller.
// ------------------------------------------------------------------------
hipError_t launch_pack_weights(const float* W, const Shape& s, uint8_t* Wq,
                               hipStream_t st);
hipError_t launch_pack_weights_q(const int8_t* q, const uint16_t* d16,
                                 const Shape& s, uint8_t* Wq, hipStream_t st);
hipError_t launch_unpack_weights(const uint8_t* Wq, const Shape& s, int8_t* q,
                                 uint16_t* d16, hipStream_t st);
// n_slots (a multiple of 16) is the slot count of the buffer Xq.
hipError_t launch_quantize_acts(const float* X, int n_rows, const Shape& s,
                                uint8_t* Xq, int n_slots, hipStream_t st);

// Matmul tiling: chosen from (N, K) only, so that the fp32 summation order
// of every output never depends on the live batch.
struct Tiling {
    int rg;           // row groups of 16 rows per wave (MFMA engine, one workgroup per row block)
    int rg_split;     // the same when the splits run as separate workgroups
    int splits;       // K splits (level 2 of the summation tree)
    int kw;           // wave slices per split (level 1)
    int ring;         // chunks in flight per wave (1, 2 or 4); no effect on the sums
    bool nt_weights;  // non-temporal loads for the weight stream
    // seq: one wave per row block evaluates every split in turn (kw == 1),
    // instead of a wave per split; split_from: in the split execution, the
    // row groups before it run that way and only the rest as split
    // workgroups.  Neither changes the sums.
    bool seq;
    int64_t split_from;
};
Tiling choose_tiling(const Shape& s);

// Pos-vector RoPE in place on rows of Y (see q8_rope.hip).  Arguments are
// validated by the caller.
hipError_t launch_rope_multi(float* Y, int n_rows, int64_t row_stride, const int32_t* pos,
                             int n_heads, int head_dim, double base, hipStream_t st);
// Workspace a split execution needs (0: the shape is not split).
size_t workspace_bytes(const Shape& s, const Tiling& t);

// The MFMA engine's launch for one call, decided from the shape, the tiling,
// the slot buffer's width and whether the splits run through a workspace
// (the fused entry point adds its producer workgroups and keeps 4 chunks in
// flight).
struct MmPlan {
    int rg;              // row groups per wave
    int ct;              // 16-slot column tiles
    int ring;            // chunks in flight per wave
    int splits, kw;      // the tree: splits (level 2), wave slices per split (level 1)
    bool split;          // splits as separate workgroups, meeting in the workspace
    int n_rb;            // row blocks of rg row groups
    int n_whole;         // leading row blocks run by one wave that takes every split in turn
    int waves;           // waves per workgroup
    int64_t workgroups;
    size_t lds_bytes;    // dynamic LDS per workgroup
};
// false: the slot width or the tiling cannot be launched.
bool plan_matmul(const Shape& s, const Tiling& t, int n_slots, bool with_workspace,
                 MmPlan& p);
// Workspace of the fused pre-quantise + matmul: 64 KB of counters and flags
// (16 pages of 4 KB), then workspace_bytes().  The uint32 at byte
// kFusedTimeoutsOffset counts the matmul workgroups whose bounded wait ran
// out; the library never clears it.
constexpr size_t kFusedFlagBytes = 64 * 1024;
constexpr size_t kFusedTimeoutsOffset = 256;
// Polls of the fused path's bounded wait (each followed by a short sleep).
constexpr int kFusedMaxSpins = 1 << 22;

// Host checks shared by the matmul entry points: a valid shape, 1 <= n_live
// <= 16, and non-null, aligned pointers.
bool matmul_args_ok(const void* Wq, const void* Xq, const int32_t* batch_index, int n_live,
                    int64_t N, int64_t K, const float* Y);

#ifdef Q8_TIMELINE
// Timeline build: the record buffer of the following matmul launches (null
// or waves <= 0: none).
void set_timeline(uint64_t* buf, int64_t waves);
#endif

enum class Engine { kMfma, kDot4 };
// workspace: nullptr for the single-workgroup evaluation of the tree, or a
// zero-initialised buffer of workspace_bytes() for the split execution.
// n_slots: slots of the buffer Xq (16; 32, 48 or 64 only with the MFMA
// engine and no workspace).
hipError_t launch_matmul(Engine e, const uint8_t* Wq, const uint8_t* Xq,
                         int n_slots, const int32_t* batch_index, int n_live,
                         const Shape& s, const Tiling& t, float* Y,
                         void* workspace, hipStream_t st);
// Pre-quantise X [n_rows][K] into the 16-slot buffer Xq and run the matmul,
// in one launch (MFMA engine).  workspace: kFusedFlagBytes of counters
// followed by workspace_bytes() for the split execution, all zero before
// the first call and left zero by every call (but the timeout word).
// max_spins bounds each matmul workgroup's wait for the slots; quantize =
// false launches no producers at all (the wait can then only run out).
hipError_t launch_matmul_fused(const uint8_t* Wq, const float* X, int n_rows,
                               uint8_t* Xq, const int32_t* batch_index, int n_live,
                               const Shape& s, const Tiling& t, float* Y,
                               void* workspace, int max_spins, bool quantize,
                               hipStream_t st);

}  // namespace q8
