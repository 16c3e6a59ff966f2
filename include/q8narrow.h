/*
 * q8narrow.h -- narrow-batch q8_0 decode matmul for AMD Instinct MI355X
 * (gfx950): the C ABI.
 *
 * The operation.  "Batched decode: co-decode N live sessions in one GPU pass"
 * (antirez/ds4 PR #530), section "Why it's worth it -- the narrow-batch
 * matmul", and its commit "CUDA: narrow-batch q8_0 matmul for 2-4 token
 * decode": in memory-bound decode, a weight matrix stored as q8_0 blocks of
 * 32 weights is read from memory once per step and each block is dotted
 * against the pre-quantised activation blocks of every live token.  For a live
 * batch of n_live tokens gathered through batch_index from a fixed buffer of
 * 16 activation slots ("[feature] Enable Dynamic Batching" (quic/
 * efficient-transformers PR #1305), section "Objective"; "dynamic public
 * batch (1..16) for Qwen3-14B decode" (hw-native-sys/pypto-lib PR #841),
 * commit message: the live batch 1..16 against a fixed padded width):
 *
 *     S[t,n,b] = sum_{i<32} qw[n,32b+i] * qx[batch_index[t],32b+i]  (int32)
 *     Y[t,n]   = sum_b S[t,n,b] * dw[n,b] * dx[batch_index[t],b]     (fp32)
 *
 * q8_0 block (the pages name it but do not spell it out; this is the GGUF
 * reading): 32 int8 values and one binary16 scale d = absmax/127, with
 * q = clamp(round_half_away(x/d), -127, 127) using the binary32 d and IEEE
 * division; an all-zero block stores d = +0 and q = 0.
 *
 * Conventions for every entry point:
 *   - Pointers named W, X, Y, Wq, Xq, q, d16, batch_index are DEVICE
 *     pointers owned by the caller; the library allocates nothing and keeps
 *     no state beyond cached device properties.
 *   - Work is enqueued on `stream` (0 = the null stream) and is asynchronous:
 *     no host synchronisation happens inside any call.  Calls are
 *     thread-safe; calls that write the same buffer must be ordered by the
 *     caller.
 *   - Arguments are validated on the host before any HIP call; a rejected
 *     call returns Q8_ERR_INVALID_ARG and enqueues nothing.  A device that
 *     is not gfx950 gives Q8_ERR_UNSUPPORTED; a launch failure reported by
 *     the HIP runtime gives Q8_ERR_HIP.  The library never aborts.
 *   - Shapes: N >= 1 output features, K >= 32 input features with K % 32 == 0,
 *     K < 2^24, and the matrix padded to whole groups of 16 rows and 256
 *     columns holds at most 2^34 values (17 GB packed; every launch then
 *     stays below 2^32 threads).  Any other shape is an invalid argument.
 *   - Alignment: W, X, Wq, Xq 16 bytes; q 8 bytes; Y, batch_index 4 bytes;
 *     d16 2 bytes.  A null or misaligned pointer is an invalid argument.
 */
#ifndef Q8NARROW_H
#define Q8NARROW_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q8_BLOCK 32     /* values per q8_0 block */
#define Q8_MAX_SLOTS 16   /* activation slots in the padded buffer */
#define Q8_MAX_COLUMNS 64 /* slots of a multi-column buffer (q8_matmul_multi) */

typedef enum q8_status {
    Q8_OK = 0,
    Q8_ERR_INVALID_ARG = 1,
    Q8_ERR_UNSUPPORTED = 2,
    Q8_ERR_HIP = 3,
    Q8_ERR_TOO_LARGE = 4 /* the shape needs more than a fixed buffer holds */
} q8_status;

/* Which int8 dot engine the matmul uses (all give bit-identical Y). */
typedef enum q8_path {
    Q8_PATH_AUTO = 0, /* the library's choice (matrix cores) */
    Q8_PATH_MFMA = 1, /* v_mfma_i32_16x16x32_i8: 16 rows x 16 tokens per block */
    Q8_PATH_DOT4 = 2  /* v_dot4 int8 dot products, one row per lane */
} q8_path;

/* ------------------------------------------------------------------ sizes */

/* Bytes of the packed weight buffer for an N x K matrix; 0 if the shape is
 * invalid.  The packed layout is private to the library (it is tiled for
 * the matmul kernels); use q8_unpack_weights to read it back. */
size_t q8_packed_weight_bytes(int64_t N, int64_t K);

/* Bytes of an activation slot buffer for K inputs; 0 if K is invalid.
 *
 * The slot buffer holds Q8_MAX_SLOTS quantised activation rows (slots).  Its
 * layout is the packed layout of a Q8_MAX_SLOTS x K weight matrix whose row s
 * is slot s: q8_quantize_acts fills it from fp32 rows, and q8_pack_weights_q /
 * q8_unpack_weights with N = Q8_MAX_SLOTS write or read all slots in
 * canonical q8_0 form.  Equal to q8_packed_weight_bytes(Q8_MAX_SLOTS, K). */
size_t q8_act_buffer_bytes(int64_t K);

/* -------------------------------------------------------------- packing */

/* Quantise fp32 weights W [N][K] (row-major) to q8_0 and
 * write them in the packed layout to Wq (q8_packed_weight_bytes(N, K)
 * bytes).  Offline, once per matrix.
 * Same quantisation rule as above, bit-exact with the definition. */
q8_status q8_pack_weights(const float* W, int64_t N, int64_t K, void* Wq,
                          hipStream_t stream);

/* Pack already-quantised canonical q8_0 weights: q int8 [N][K] and d16
 * binary16 bits [N][K/32], both row-major.  Any int8 value, -128 included,
 * and any finite scale are accepted. */
q8_status q8_pack_weights_q(const int8_t* q, const uint16_t* d16, int64_t N,
                            int64_t K, void* Wq, hipStream_t stream);

/* Read a packed buffer back into canonical q [N][K] and d16 [N][K/32]. */
q8_status q8_unpack_weights(const void* Wq, int64_t N, int64_t K, int8_t* q,
                            uint16_t* d16, hipStream_t stream);

/* --------------------------------------------------------- activations */

/* Pre-quantise activations ("preq"; same page, same section): fp32 rows
 * X [n_rows][K] (row-major) go to slots 0..n_rows-1 of the slot buffer Xq,
 * block by block with the q8_0 rule.
 * Slots n_rows..15 are left untouched.  1 <= n_rows <= Q8_MAX_SLOTS. */
q8_status q8_quantize_acts(const float* X, int n_rows, int64_t K, void* Xq,
                           hipStream_t stream);

/* ------------------------------------------------------------- matmul */

/* Y[t][n] for t < n_live, n < N (fp32, row-major [n_live][N], overwritten,
 * 4-byte aligned).  Wq: packed weights of the N x K matrix.  Xq: an
 * activation slot buffer for K.  batch_index: int32 [n_live] device array;
 * token t uses slot batch_index[t]; entries may repeat and come in any
 * order.  1 <= n_live <= Q8_MAX_SLOTS.
 *
 * Each weight block is read from memory once per call and used for every
 * live token.  The fp32 summation order (a fixed tree over K: blocks in
 * order within a slice, slices in order within a split, splits in order)
 * depends only on (N, K), never on n_live or on the other tokens, so row t
 * of Y is bit-identical to a call with n_live = 1 and batch_index =
 * {batch_index[t]}.
 *
 * A batch_index entry outside [0, 16) cannot be checked on the host without
 * a synchronisation; it is not read through: that token's row of Y is set
 * to quiet NaN. */
q8_status q8_matmul_narrow(const void* Wq, const void* Xq,
                           const int32_t* batch_index, int n_live, int64_t N,
                           int64_t K, float* Y, hipStream_t stream);

/* As q8_matmul_narrow, with an explicit choice of int8 dot engine (for
 * comparing the two; both give bit-identical results). */
q8_status q8_matmul_narrow_path(const void* Wq, const void* Xq,
                                const int32_t* batch_index, int n_live,
                                int64_t N, int64_t K, float* Y,
                                hipStream_t stream, q8_path path);

/* ---------------------------------------------- workspace execution */

/* Bytes of workspace q8_matmul_narrow_ws needs for an N x K matrix; 0 when
 * the shape is not split across workgroups (then no workspace is needed) or
 * the shape is invalid. */
size_t q8_matmul_workspace_bytes(int64_t N, int64_t K);

/* q8_matmul_narrow, executed with the K splits of row blocks spread over
 * separate workgroups: every row block for long rows (K >= 8192), which
 * balances small-N shapes over the whole GPU (except when the row blocks of
 * two row groups of 16 rows number 205..256: those shapes fill 80-100% of
 * the CUs with one workgroup each, which adds its 4 K ranges in LDS, and
 * need no workspace); for 1024..4400 row groups of
 * 16 rows that are not a multiple of the GPU's 256 CUs, only the last
 * (row groups mod 256) row blocks, so that every CU streams the same bytes.
 * The splits meet through `workspace` (device memory, 256-byte aligned, at
 * least q8_matmul_workspace_bytes(N, K) bytes): each split publishes its
 * partial sums, and the last to arrive adds them in split order.  The result
 * is bit-identical to q8_matmul_narrow on the same arguments.
 *
 * The workspace must be zero-filled before its first use.  Every completed
 * call leaves it ready for the next one, on a matrix of the same shape or of
 * any other (as long as the workspace is large enough for it): the arrival
 * counters are back at zero, and the partial sums left behind sit where no
 * shape keeps a counter.  A workspace must not be shared by calls that can
 * run at the same time (calls on one stream are fine), nor between this
 * entry point and q8_matmul_narrow_fused, whose workspace is laid out
 * differently, without being zero-filled again in between.
 * workspace may be NULL when q8_matmul_workspace_bytes(N, K) is 0.  A
 * workspace that is missing, misaligned or too small is an invalid
 * argument. */
q8_status q8_matmul_narrow_ws(const void* Wq, const void* Xq,
                              const int32_t* batch_index, int n_live,
                              int64_t N, int64_t K, float* Y, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------- launch plan */

/* The MFMA engine's launch for an N x K matrix, as the matmul entry points
 * enqueue it: q8_matmul_narrow (with_workspace = 0, n_slots = 16),
 * q8_matmul_narrow_ws and q8_matmul_narrow_noalloc (with_workspace = 1,
 * n_slots = 16), q8_matmul_multi (with_workspace = 0, n_slots 32, 48 or 64).
 * Everything here follows from (N, K, n_slots) alone, never from the live
 * batch, which is what keeps a column's bits independent of it.  The fields
 * name the fixed summation tree (a wave adds its blocks in order, the
 * slices of a split are added in order, then the splits in order) and how
 * the launch evaluates it.
 * The fused entry point launches the with_workspace = 1 plan plus its
 * producer workgroups, at 4 chunks in flight.  Host only: no device call. */
typedef struct {
    int32_t row_groups_per_wave;   /* row groups of 16 rows each wave streams */
    int32_t column_tiles;          /* n_slots / 16 */
    int32_t chunks_in_flight;      /* weight chunks (1 KB per row group) per wave */
    int32_t k_splits;              /* splits of K (the tree's level 2) */
    int32_t slices_per_split;      /* wave slices of a split (level 1) */
    int32_t split_workgroups;      /* 1: the splits of some row blocks run as
                                      separate workgroups meeting in the workspace */
    int32_t whole_row_workgroups;  /* leading workgroups of one wave that
                                      evaluates every split of its row block in turn */
    int32_t waves_per_workgroup;   /* of 64 lanes */
    int64_t workgroups;
    int64_t lds_bytes;             /* dynamic LDS per workgroup */
} q8_launch_info;

/* Fills *info.  Q8_ERR_INVALID_ARG for a null info, an invalid shape, an
 * n_slots other than 16, 32, 48 or 64, or with_workspace other than 0 or
 * 1 (1 only with n_slots = 16); else Q8_OK. */
q8_status q8_matmul_launch_info(int64_t N, int64_t K, int n_slots, int with_workspace,
                                q8_launch_info* info);

/* ----------------------------------------------- no-allocation variant */

/* Bytes of the device array behind q8_matmul_narrow_noalloc (8 MiB). */
#define Q8_NOALLOC_SCRATCH_BYTES (8u << 20)

/* For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Computes exactly what q8_matmul_narrow_ws computes (the same
 * kernels, the same bits), with the workspace taken from a static device
 * array of Q8_NOALLOC_SCRATCH_BYTES that the library holds on every device
 * it runs on until the process ends.  The call allocates nothing: no
 * hipMalloc, no hipFree, no allocating library routine.
 *
 * Limit: shapes whose q8_matmul_workspace_bytes(N, K) exceeds
 * Q8_NOALLOC_SCRATCH_BYTES return Q8_ERR_TOO_LARGE and enqueue nothing
 * (8 MiB holds the split records of up to 1927 row groups of 16 rows, i.e.
 * N <= 30832 for the long rows (K >= 8192) whose row groups are all split;
 * other shapes split at most 128 row groups or none).
 *
 * The first call on a device takes the array's device address and enqueues
 * a small kernel on `stream` that zero-fills it; make that first call
 * outside stream capture.  Every completed call leaves the array ready for
 * the next, on any shape.  All calls on one device share the one array: calls
 * that can run at the same time on one device (other streams, other host
 * threads without ordering) race and give wrong results; calls ordered on
 * one stream are fine.  Other arguments and errors as q8_matmul_narrow. */
q8_status q8_matmul_narrow_noalloc(const void* Wq, const void* Xq,
                                   const int32_t* batch_index, int n_live, int64_t N,
                                   int64_t K, float* Y, hipStream_t stream);

/* ------------------------------------------- fused pre-quantisation */

/* Bytes of workspace q8_matmul_narrow_fused needs for an N x K matrix (64 KB
 * of counters and flags, then q8_matmul_workspace_bytes(N, K)); 0 if the
 * shape is invalid. */
size_t q8_matmul_fused_workspace_bytes(int64_t N, int64_t K);

/* Byte offset, in a fused workspace, of a uint32 that counts the matmul
 * workgroups whose wait for the published slots ran out (see below).  The
 * library only ever adds to it; it is zero after the caller's zero-fill. */
#define Q8_FUSED_TIMEOUTS_OFFSET 256

/* q8_quantize_acts(X, n_rows, K, Xq) followed by q8_matmul_narrow_ws(Wq, Xq,
 * batch_index, n_live, N, K, Y, workspace) in one launch, with the same
 * results: Xq receives the same bits as q8_quantize_acts would write and Y
 * the same bits as the matmul.  "Batched decode: co-decode N live sessions
 * in one GPU pass" (antirez/ds4 PR #530), commit "CUDA: add pos-vector RoPE
 * tail variants", measures a couple of microseconds per extra launch, which
 * adds up over a decode step; this removes the pre-quantiser's launch (the
 * activations are small next to the weights: section "Why it's worth it --
 * the narrow-batch matmul").  A few workgroups of the launch quantise X and
 * publish the slots; the matmul workgroups stream their first weights while
 * they wait for them.
 *
 * The wait is bounded.  Should it ever run out (it cannot in a normal call:
 * the quantising workgroups are dispatched first and wait on nothing), the
 * workgroup writes quiet NaN over every output row it owns and adds one to
 * the uint32 at byte Q8_FUSED_TIMEOUTS_OFFSET of the workspace, and the
 * kernel still finishes; the call itself returns Q8_OK, since nothing is
 * known on the host without a synchronisation.
 *
 * workspace: device memory, 256-byte aligned, at least
 * q8_matmul_fused_workspace_bytes(N, K) bytes, zero-filled before its first
 * use.  Every completed call leaves its counters and flags at zero again (as
 * with q8_matmul_narrow_ws, partial sums left behind are never taken for
 * counters), so it may serve matrices of any shape in turn.  It must not be
 * shared by calls that can run at the same time.  1 <= n_rows, n_live <= Q8_MAX_SLOTS;
 * X fp32 [n_rows][K], 16-byte aligned. */
q8_status q8_matmul_narrow_fused(const void* Wq, const float* X, int n_rows, void* Xq,
                                 const int32_t* batch_index, int n_live, int64_t N,
                                 int64_t K, float* Y, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* q8_matmul_narrow_fused with the bound of the wait given: each matmul
 * workgroup polls for the published slots at most max_spins times (1 ..
 * 2^30; q8_matmul_narrow_fused uses 2^22, each poll followed by a short
 * sleep).  quantize = 0 launches no quantising workgroups at all, so the
 * slots are neither written nor published and every wait runs out: a way to
 * exercise the failure path from the host (every output NaN, the timeout
 * word raised, the workspace rearmed for the next call).  quantize = 1 is
 * q8_matmul_narrow_fused.  Other arguments and errors as there. */
q8_status q8_matmul_narrow_fused_bounded(const void* Wq, const float* X, int n_rows, void* Xq,
                                         const int32_t* batch_index, int n_live, int64_t N,
                                         int64_t K, float* Y, void* workspace,
                                         size_t workspace_bytes, int max_spins, int quantize,
                                         hipStream_t stream);

/* ------------------------------------------------- multi-token columns */

/* Several tokens per sequence in one step: "[feature] Enable Dynamic
 * Batching", section "Assumptions and limitations" (dynamic batching
 * combined with multi-spec speculative decoding: batch on one axis, the
 * speculative length on the other, e.g. b=2, k=3 -> input_ids (2, 4)).  With
 * n_seq sequences of k+1 tokens each, a weight block meets n_seq*(k+1)
 * activation columns, up to Q8_MAX_COLUMNS here, and is still read from
 * memory once.
 *
 * A multi-column slot buffer holds n_slots = 16, 32, 48 or 64 slots in the
 * packed layout of an n_slots x K matrix (with n_slots = 16 it is exactly
 * the q8_act_buffer_bytes buffer).  Returns its size in bytes, 0 if K or
 * n_slots is invalid. */
size_t q8_act_buffer_bytes_n(int64_t K, int n_slots);

/* q8_quantize_acts for an n_slots buffer: rows X [n_rows][K] go to slots
 * 0..n_rows-1; the others are left untouched.  1 <= n_rows <= n_slots. */
q8_status q8_quantize_acts_n(const float* X, int n_rows, int64_t K, void* Xq,
                             int n_slots, hipStream_t stream);

/* q8_matmul_narrow over an n_slots buffer: Y [n_live][N], token t uses slot
 * batch_index[t] in [0, n_slots); 1 <= n_live <= n_slots.  The summation
 * tree is the one of q8_matmul_narrow (it depends on (N, K) only), so a
 * column is bit-identical to q8_matmul_narrow's for the same slot contents,
 * and to this call with n_live = 1.  A batch_index entry outside
 * [0, n_slots) gives a NaN row. */
q8_status q8_matmul_multi(const void* Wq, const void* Xq, int n_slots,
                          const int32_t* batch_index, int n_live, int64_t N,
                          int64_t K, float* Y, hipStream_t stream);

/* ------------------------------------------------------ pos-vector RoPE */

/* Rotary position embedding with one position per row, in place, for the
 * rows a batched QKV projection produces.  "Batched decode: co-decode N
 * live sessions in one GPU pass" (antirez/ds4 PR #530), commit "CUDA: add
 * pos-vector RoPE tail variants": each row (token) has its own position,
 * read from a small per-row array, and each row's result is bitwise the one
 * a single-row call would give.
 *
 * Y: fp32 rows, n_rows of them, row_stride floats apart (e.g. the [n_live][N]
 * output of q8_matmul_narrow, row_stride = N); the first n_heads * head_dim
 * columns are the heads to rotate (e.g. the query and key heads), the rest
 * are left untouched.  pos: int32 [n_rows] device array.  In each head,
 * values i and i + head_dim/2 (i < head_dim/2) are rotated by the angle
 * pos[t] * base^(-2i/head_dim) (the rotate-half pairing); the angle, its
 * sine and cosine and the rotation are computed in double and rounded once
 * to fp32.
 *
 * 1 <= n_rows <= Q8_MAX_COLUMNS; n_heads >= 1; head_dim even, 2..1024;
 * n_heads * head_dim <= row_stride; n_rows * n_heads * head_dim <= 2^32;
 * n_rows * row_stride <= 2^40; 1 < base < 1e30; Y and pos 4-byte aligned. */
q8_status q8_rope_multi(float* Y, int n_rows, int64_t row_stride, const int32_t* pos,
                        int n_heads, int head_dim, double base, hipStream_t stream);

/* --------------------------------------------------------- measurement */

/* A plain read-only streaming kernel: reads every 16-byte unit of buf once
 * (non-temporal loads, a grid-stride loop of 2048 x 256 threads) and
 * computes nothing else.  Its rate over a large buffer is the measured HBM
 * read ceiling against which the matmul's achieved bandwidth is set (the
 * measurement section of the hot-path scope asks for it beside the vendor
 * peak).  Each thread XORs the words it reads and writes sink[thread %
 * 1024] only if that XOR equals 0x9E3779B9, so the loads cannot be dropped
 * and, for ordinary data, nothing is written.
 *
 * buf: device, 16-byte aligned, bytes a positive multiple of 16 (at most
 * 2^40); sink: device uint32 [1024], caller-owned.  Stream-ordered. */
q8_status q8_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

/* ---------------------------------------------------------------- misc */

/* 1 if the current HIP device is gfx950, 0 if not or if none is usable. */
int q8_device_supported(void);

/* A static string naming a status code. */
const char* q8_status_str(q8_status status);

#ifdef __cplusplus
}
#endif

#endif /* Q8NARROW_H */
