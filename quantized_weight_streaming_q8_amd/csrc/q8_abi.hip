// q8_abi.hip -- the extern "C" entry points of libq8narrow.so (see
// include/q8narrow.h for the contract).
//
// Every entry point validates its arguments on the host before making any
// HIP call, in the spirit of "[feature] Enable Dynamic Batching", section
// "Assumptions and limitations" (reject an invalid combination early with a
// clear error) and of "dynamic public batch (1..16) for Qwen3-14B decode",
// commit message (the live batch must satisfy 1 <= batch <= pad).  Then it
// checks the device (gfx950 only) and enqueues kernels on the caller's
// stream.  Nothing is allocated and nothing synchronises.

#include "q8narrow.h"
#include "q8_internal.h"
#include "q8_measure.h"
#ifdef Q8_TIMELINE
#include "q8timeline.h"
#endif

#include <atomic>
#include <cstring>

namespace {

constexpr int64_t kMaxK = int64_t(1) << 24;
// Values of the matrix padded to whole row groups (16 rows) and super-chunks
// (256 values).  The packer runs one thread per 8 padded values, and a
// launch must stay below 2^32 threads; 2^34 values is 17 GB packed.
constexpr int64_t kMaxPaddedNK = int64_t(1) << 34;

bool valid_shape(int64_t N, int64_t K) {
    if (N < 1 || K < Q8_BLOCK || K % Q8_BLOCK != 0 || K >= kMaxK) return false;
    const int64_t Kp = (K + 255) / 256 * 256;
    return N <= kMaxPaddedNK / Kp && (N + 15) / 16 * 16 <= kMaxPaddedNK / Kp;
}

bool valid_slots(int n_slots) {
    return n_slots >= Q8_MAX_SLOTS && n_slots <= Q8_MAX_COLUMNS && n_slots % Q8_MAX_SLOTS == 0;
}

bool aligned(const void* p, uintptr_t a) {
    return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) == 0;
}

// Per-device cache of "is this a gfx950": 0 unknown, 1 yes, 2 no.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

int current_device_ok() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < kMaxDevices) {
        const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
        if (c) return c == 1;
    }
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return 0;
    const int ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 &&
                   (prop.gcnArchName[6] == '\0' || prop.gcnArchName[6] == ':');
    if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
    return ok;
}

q8_status from_hip(hipError_t e) { return e == hipSuccess ? Q8_OK : Q8_ERR_HIP; }

}  // namespace

namespace q8 {

bool matmul_args_ok(const void* Wq, const void* Xq, const int32_t* batch_index, int n_live,
                    int64_t N, int64_t K, const float* Y) {
    return valid_shape(N, K) && n_live >= 1 && n_live <= Q8_MAX_SLOTS && aligned(Wq, 16) &&
           aligned(Xq, 16) && aligned(batch_index, 4) && aligned(Y, 4);
}

}  // namespace q8

extern "C" {

size_t q8_packed_weight_bytes(int64_t N, int64_t K) {
    if (!valid_shape(N, K)) return 0;
    const q8::Shape s = q8::make_shape(N, K);
    return (size_t)(s.q_bytes + s.d_bytes);
}

size_t q8_act_buffer_bytes(int64_t K) {
    return q8_packed_weight_bytes(Q8_MAX_SLOTS, K);
}

size_t q8_act_buffer_bytes_n(int64_t K, int n_slots) {
    if (!valid_slots(n_slots)) return 0;
    return q8_packed_weight_bytes(n_slots, K);
}

q8_status q8_pack_weights(const float* W, int64_t N, int64_t K, void* Wq,
                          hipStream_t stream) {
    if (!valid_shape(N, K) || !aligned(W, 16) || !aligned(Wq, 16)) return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    return from_hip(q8::launch_pack_weights(W, s, static_cast<uint8_t*>(Wq), stream));
}

q8_status q8_pack_weights_q(const int8_t* q, const uint16_t* d16, int64_t N,
                            int64_t K, void* Wq, hipStream_t stream) {
    if (!valid_shape(N, K) || !aligned(q, 8) || !aligned(d16, 2) || !aligned(Wq, 16))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    return from_hip(q8::launch_pack_weights_q(q, d16, s, static_cast<uint8_t*>(Wq), stream));
}

q8_status q8_unpack_weights(const void* Wq, int64_t N, int64_t K, int8_t* q,
                            uint16_t* d16, hipStream_t stream) {
    if (!valid_shape(N, K) || !aligned(Wq, 16) || !aligned(q, 8) || !aligned(d16, 2))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    return from_hip(q8::launch_unpack_weights(static_cast<const uint8_t*>(Wq), s, q, d16, stream));
}

q8_status q8_quantize_acts_n(const float* X, int n_rows, int64_t K, void* Xq,
                             int n_slots, hipStream_t stream) {
    if (!valid_shape(1, K) || !valid_slots(n_slots) || n_rows < 1 || n_rows > n_slots ||
        !aligned(X, 16) || !aligned(Xq, 16))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(1, K);
    return from_hip(q8::launch_quantize_acts(X, n_rows, s, static_cast<uint8_t*>(Xq), n_slots,
                                             stream));
}

q8_status q8_quantize_acts(const float* X, int n_rows, int64_t K, void* Xq,
                           hipStream_t stream) {
    return q8_quantize_acts_n(X, n_rows, K, Xq, Q8_MAX_SLOTS, stream);
}

q8_status q8_matmul_narrow_path(const void* Wq, const void* Xq,
                                const int32_t* batch_index, int n_live,
                                int64_t N, int64_t K, float* Y,
                                hipStream_t stream, q8_path path) {
    if (!q8::matmul_args_ok(Wq, Xq, batch_index, n_live, N, K, Y)) return Q8_ERR_INVALID_ARG;
    if (path != Q8_PATH_AUTO && path != Q8_PATH_MFMA && path != Q8_PATH_DOT4)
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    const q8::Tiling t = q8::choose_tiling(s);
    const q8::Engine e = path == Q8_PATH_DOT4 ? q8::Engine::kDot4 : q8::Engine::kMfma;
    return from_hip(q8::launch_matmul(e, static_cast<const uint8_t*>(Wq),
                                      static_cast<const uint8_t*>(Xq), Q8_MAX_SLOTS,
                                      batch_index, n_live, s, t, Y, nullptr, stream));
}

q8_status q8_matmul_narrow(const void* Wq, const void* Xq,
                           const int32_t* batch_index, int n_live, int64_t N,
                           int64_t K, float* Y, hipStream_t stream) {
    return q8_matmul_narrow_path(Wq, Xq, batch_index, n_live, N, K, Y, stream,
                                 Q8_PATH_AUTO);
}

size_t q8_matmul_workspace_bytes(int64_t N, int64_t K) {
    if (!valid_shape(N, K)) return 0;
    const q8::Shape s = q8::make_shape(N, K);
    return q8::workspace_bytes(s, q8::choose_tiling(s));
}

q8_status q8_matmul_launch_info(int64_t N, int64_t K, int n_slots, int with_workspace,
                                q8_launch_info* info) {
    if (info == nullptr || !valid_shape(N, K)) return Q8_ERR_INVALID_ARG;
    if (with_workspace != 0 && (with_workspace != 1 || n_slots != Q8_MAX_SLOTS))
        return Q8_ERR_INVALID_ARG;
    const q8::Shape s = q8::make_shape(N, K);
    const q8::Tiling t = q8::choose_tiling(s);
    q8::MmPlan p;
    if (!q8::plan_matmul(s, t, n_slots, with_workspace == 1 && q8::workspace_bytes(s, t) > 0, p))
        return Q8_ERR_INVALID_ARG;
    info->row_groups_per_wave = p.rg;
    info->column_tiles = p.ct;
    info->chunks_in_flight = p.ring;
    info->k_splits = p.splits;
    info->slices_per_split = p.kw;
    info->split_workgroups = p.split ? 1 : 0;
    info->whole_row_workgroups = p.n_whole;
    info->waves_per_workgroup = p.waves;
    info->workgroups = p.workgroups;
    info->lds_bytes = (int64_t)p.lds_bytes;
    return Q8_OK;
}

q8_status q8_matmul_narrow_ws(const void* Wq, const void* Xq,
                              const int32_t* batch_index, int n_live, int64_t N,
                              int64_t K, float* Y, void* workspace,
                              size_t workspace_size, hipStream_t stream) {
    if (!q8::matmul_args_ok(Wq, Xq, batch_index, n_live, N, K, Y)) return Q8_ERR_INVALID_ARG;
    const q8::Shape s = q8::make_shape(N, K);
    const q8::Tiling t = q8::choose_tiling(s);
    const size_t need = q8::workspace_bytes(s, t);
    if (need > 0 && (!aligned(workspace, 256) || workspace_size < need)) return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    return from_hip(q8::launch_matmul(q8::Engine::kMfma, static_cast<const uint8_t*>(Wq),
                                      static_cast<const uint8_t*>(Xq), Q8_MAX_SLOTS,
                                      batch_index, n_live, s, t, Y,
                                      need > 0 ? workspace : nullptr, stream));
}

size_t q8_matmul_fused_workspace_bytes(int64_t N, int64_t K) {
    if (!valid_shape(N, K)) return 0;
    const q8::Shape s = q8::make_shape(N, K);
    return q8::kFusedFlagBytes + q8::workspace_bytes(s, q8::choose_tiling(s));
}

q8_status q8_matmul_narrow_fused_bounded(const void* Wq, const float* X, int n_rows, void* Xq,
                                         const int32_t* batch_index, int n_live, int64_t N,
                                         int64_t K, float* Y, void* workspace,
                                         size_t workspace_size, int max_spins, int quantize,
                                         hipStream_t stream) {
    if (!valid_shape(N, K) || n_rows < 1 || n_rows > Q8_MAX_SLOTS || n_live < 1 ||
        n_live > Q8_MAX_SLOTS || !aligned(Wq, 16) || !aligned(X, 16) || !aligned(Xq, 16) ||
        !aligned(batch_index, 4) || !aligned(Y, 4) || max_spins < 1 || max_spins > (1 << 30) ||
        (quantize != 0 && quantize != 1))
        return Q8_ERR_INVALID_ARG;
    const size_t need = q8_matmul_fused_workspace_bytes(N, K);
    if (!aligned(workspace, 256) || workspace_size < need) return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    return from_hip(q8::launch_matmul_fused(static_cast<const uint8_t*>(Wq), X, n_rows,
                                            static_cast<uint8_t*>(Xq), batch_index, n_live, s,
                                            q8::choose_tiling(s), Y, workspace, max_spins,
                                            quantize != 0, stream));
}

q8_status q8_matmul_narrow_fused(const void* Wq, const float* X, int n_rows, void* Xq,
                                 const int32_t* batch_index, int n_live, int64_t N,
                                 int64_t K, float* Y, void* workspace,
                                 size_t workspace_size, hipStream_t stream) {
    return q8_matmul_narrow_fused_bounded(Wq, X, n_rows, Xq, batch_index, n_live, N, K, Y,
                                          workspace, workspace_size, q8::kFusedMaxSpins, 1,
                                          stream);
}

q8_status q8_matmul_multi(const void* Wq, const void* Xq, int n_slots,
                          const int32_t* batch_index, int n_live, int64_t N,
                          int64_t K, float* Y, hipStream_t stream) {
    if (!valid_shape(N, K) || !valid_slots(n_slots) || n_live < 1 || n_live > n_slots ||
        !aligned(Wq, 16) || !aligned(Xq, 16) || !aligned(batch_index, 4) || !aligned(Y, 4))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    const q8::Shape s = q8::make_shape(N, K);
    const q8::Tiling t = q8::choose_tiling(s);
    return from_hip(q8::launch_matmul(q8::Engine::kMfma, static_cast<const uint8_t*>(Wq),
                                      static_cast<const uint8_t*>(Xq), n_slots, batch_index,
                                      n_live, s, t, Y, nullptr, stream));
}

q8_status q8_rope_multi(float* Y, int n_rows, int64_t row_stride, const int32_t* pos,
                        int n_heads, int head_dim, double base, hipStream_t stream) {
    if (n_rows < 1 || n_rows > Q8_MAX_COLUMNS || n_heads < 1 || head_dim < 2 ||
        head_dim % 2 != 0 || head_dim > 1024 || row_stride < (int64_t)n_heads * head_dim ||
        row_stride > (int64_t(1) << 40) / n_rows ||
        (int64_t)n_heads * head_dim > (int64_t(1) << 32) / n_rows || !(base > 1.0) || !(base < 1e30) ||
        !aligned(Y, 4) || !aligned(pos, 4))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    return from_hip(q8::launch_rope_multi(Y, n_rows, row_stride, pos, n_heads, head_dim, base,
                                          stream));
}

q8_status q8_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
    if (buf == nullptr || sink == nullptr || bytes == 0 || bytes % 16 != 0 ||
        bytes > (size_t(1) << 40) || !aligned(buf, 16) || !aligned(sink, 4))
        return Q8_ERR_INVALID_ARG;
    if (!current_device_ok()) return Q8_ERR_UNSUPPORTED;
    return from_hip(q8::launch_stream_read(buf, (int64_t)bytes, sink, stream));
}

int q8_device_supported(void) { return current_device_ok(); }

#ifdef Q8_TIMELINE
q8_status q8_timeline_set(uint64_t* records, int64_t max_waves) {
    if (max_waves < 0 || (max_waves > 0 && (records == nullptr || !aligned(records, 8))))
        return Q8_ERR_INVALID_ARG;
    q8::set_timeline(records, max_waves);
    return Q8_OK;
}
#endif

const char* q8_status_str(q8_status status) {
    switch (status) {
        case Q8_OK: return "Q8_OK";
        case Q8_ERR_INVALID_ARG: return "Q8_ERR_INVALID_ARG";
        case Q8_ERR_UNSUPPORTED: return "Q8_ERR_UNSUPPORTED";
        case Q8_ERR_HIP: return "Q8_ERR_HIP";
        case Q8_ERR_TOO_LARGE: return "Q8_ERR_TOO_LARGE";
    }
    return "Q8_ERR_UNKNOWN";
}

}  // extern "C"
