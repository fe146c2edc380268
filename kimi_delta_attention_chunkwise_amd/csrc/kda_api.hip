// kda_api.hip -- the extern "C" entry points of libkda.so: host-side argument
// validation, workspace sizing and dispatch to the gfx950 kernels.  Nothing
// here allocates memory.  State kept between calls: the device address of the
// no-allocation forward's static scratch array, per device (the one auxiliary
// stream of the long-sequence forward lives with its launcher).
#include "kda.h"
#include "kda_internal.h"

#include <initializer_list>
#include <mutex>

namespace {

// Workspace of kda_chunk_fwd_noalloc: one static array per device, in place of
// the caller's workspace.  In host code `scratch` is only a stand-in for the
// symbol: its device address (different on every device) comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to the kernels.
static __device__ __align__(256) uint8_t scratch[KDA_NOALLOC_SCRATCH_BYTES];
static_assert(KDA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch keeps records 256-byte aligned");

constexpr int kScratchDevices = kda::kMaxDevices;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kScratchDevices];

// Device address of the current device's scratch array (taken at the first
// call on that device).
hipError_t scratch_address(void **ptr)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kScratchDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (!p)
            return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

bool valid_dtype(kda_dtype dt) { return dt == KDA_F32 || dt == KDA_BF16; }

bool chunk_supported(kda_dtype dt, int dk, int dv, int chunk)
{
    if (dt == KDA_BF16)
        return dk == kda::kDK && dv == kda::kDV && chunk == kda::kChunk;
    if (dt == KDA_F32)
        return dk == 16 && dv == 16 && chunk == 16;
    return false;
}

bool bwd_supported(kda_dtype dt, int dk, int dv, int chunk)
{
    return chunk_supported(dt, dk, dv, chunk);
}

bool decode_supported(kda_dtype dt, int dk, int dv)
{
    return valid_dtype(dt) && dk == dv && (dk == 16 || dk == 128);
}

// Number of chunk slots per head the bf16 path uses (see seq_info).
int64_t chunk_slots(int B, int T, int N, int chunk, int varlen)
{
    if (varlen)
        return (int64_t)T / chunk + N;
    return (int64_t)B * ((T + chunk - 1) / chunk);
}

// Slots of two chunks per head (pair records).
int64_t pair_slots(int B, int T, int N, int chunk, int varlen)
{
    return chunk_slots(B, T, N, 2 * chunk, varlen);
}

bool sizes_valid(int B, int T, int N, int H, int varlen)
{
    return !(B < 1 || T < 0 || N < 0 || H < 1 || (varlen && B != 1) || (!varlen && N != B));
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// Alignment the kernels' vector accesses rely on (NULL passes): tensors 16
// bytes, beta its element, cu_seqlens / accepted 4 bytes, workspaces 256.
constexpr uintptr_t kTensorAlign = 16, kWorkspaceAlign = 256;
bool aligned_to(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }
bool tensors_aligned(std::initializer_list<const void *> ps)
{
    for (const void *p : ps)
        if (!aligned_to(p, kTensorAlign))
            return false;
    return true;
}
uintptr_t elem_bytes(kda_dtype dt) { return dt == KDA_BF16 ? 2 : 4; }

constexpr unsigned kProAll = KDA_PRO_QK_L2NORM | KDA_PRO_BETA_SIGMOID | KDA_PRO_G_SOFTPLUS;
constexpr unsigned kFwdFlags = kProAll | KDA_FWD_CHUNK_RECORDS;
static_assert(KDA_PRO_QK_L2NORM == kda::kProQK && KDA_PRO_BETA_SIGMOID == kda::kProBeta &&
                  KDA_PRO_G_SOFTPLUS == kda::kProG,
              "prologue bits agree with the kernels");

}  // namespace

extern "C" {

const char *kda_status_str(kda_status s)
{
    switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL_POINTER: return "KDA_ERR_NULL_POINTER";
    case KDA_ERR_BAD_SHAPE: return "KDA_ERR_BAD_SHAPE";
    case KDA_ERR_BAD_DTYPE: return "KDA_ERR_BAD_DTYPE";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED";
    case KDA_ERR_WORKSPACE_TOO_SMALL: return "KDA_ERR_WORKSPACE_TOO_SMALL";
    case KDA_ERR_HIP: return "KDA_ERR_HIP";
    case KDA_ERR_MISALIGNED: return "KDA_ERR_MISALIGNED";
    case KDA_ERR_SCRATCH_LIMIT: return "KDA_ERR_SCRATCH_LIMIT";
    }
    return "KDA_ERR_UNKNOWN";
}

int kda_chunk_fwd_supported(kda_dtype dt, int dk, int dv, int chunk)
{
    return chunk_supported(dt, dk, dv, chunk) ? 1 : 0;
}

int kda_decode_step_supported(kda_dtype dt, int dk, int dv)
{
    return decode_supported(dt, dk, dv) ? 1 : 0;
}

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                     kda_dtype dt, int varlen)
{
    if (!valid_dtype(dt) || !chunk_supported(dt, dk, dv, chunk) || !sizes_valid(B, T, N, H, varlen))
        return (size_t)-1;
    if (dt == KDA_F32)
        return 0;
    return (size_t)pair_slots(B, T, N, chunk, varlen) * (size_t)H * kda::kPairRecBytes;
}

size_t kda_chunk_fwd_records_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                   kda_dtype dt, int varlen)
{
    if (!valid_dtype(dt) || !chunk_supported(dt, dk, dv, chunk) || !sizes_valid(B, T, N, H, varlen))
        return (size_t)-1;
    if (dt == KDA_F32)
        return 0;
    return (size_t)chunk_slots(B, T, N, chunk, varlen) * (size_t)H * kda::kChunkRecBytes;
}

size_t kda_snapshot_slots(int B, int T, int N, int chunk, int interval, int varlen)
{
    if (B < 1 || T < 0 || N < 0 || chunk < 1 || interval < chunk || interval % chunk != 0 ||
        (varlen && B != 1) || (!varlen && N != B))
        return (size_t)-1;
    if (varlen)
        return (size_t)(T / interval) + (size_t)N;
    return (size_t)B * (size_t)(T / interval);
}

}  // extern "C"

namespace {

// The forward behind kda_chunk_fwd_ex and kda_chunk_fwd_noalloc.  noalloc:
// the workspace is the current device's static scratch array (its size is
// checked here, before anything else touches the device), and every kernel
// stays on `stream`.
kda_status chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                     const void *beta, const void *gate, const float *init_state, void *out,
                     float *final_state, float *snapshots, int snapshot_interval,
                     const int32_t *cu_seqlens, int B, int T, int N, int H, int dk, int dv,
                     int chunk, float scale, kda_dtype dt, unsigned flags, void *workspace,
                     size_t workspace_bytes, hipStream_t stream, bool noalloc)
{
    if (!valid_dtype(dt))
        return KDA_ERR_BAD_DTYPE;
    if (!chunk_supported(dt, dk, dv, chunk) || (flags & ~kFwdFlags) != 0)
        return KDA_ERR_UNSUPPORTED;
    const unsigned prologue = flags & kProAll;
    const int varlen = cu_seqlens != nullptr;
    if (B < 1 || T < 0 || N < 0 || H < 1)
        return KDA_ERR_BAD_SHAPE;
    if (varlen ? B != 1 : N != B)
        return KDA_ERR_BAD_SHAPE;
    if (snapshots && (snapshot_interval < chunk || snapshot_interval % chunk != 0))
        return KDA_ERR_BAD_SHAPE;
    const bool has_tokens = (int64_t)B * T > 0;
    if (has_tokens && (!q || !k || !v || !g || !beta || !gate || !out))
        return KDA_ERR_NULL_POINTER;
    // bf16: pair records, unless the caller keeps per-chunk records for the
    // backward or a snapshot falls inside a pair
    const bool pair = dt == KDA_BF16 && !(flags & KDA_FWD_CHUNK_RECORDS) &&
                      !(snapshots && snapshot_interval % (2 * chunk) != 0);
    const size_t need =
        pair ? kda_chunk_fwd_workspace_bytes(B, T, N, H, dk, dv, chunk, dt, varlen)
             : kda_chunk_fwd_records_bytes(B, T, N, H, dk, dv, chunk, dt, varlen);
    const int64_t n_slots =
        pair ? pair_slots(B, T, N, chunk, varlen) : chunk_slots(B, T, N, chunk, varlen);
    if (noalloc) {
        if (need > KDA_NOALLOC_SCRATCH_BYTES)
            return KDA_ERR_SCRATCH_LIMIT;
        workspace_bytes = KDA_NOALLOC_SCRATCH_BYTES;
    } else {
        if (need > 0 && !workspace)
            return KDA_ERR_NULL_POINTER;
        if (workspace_bytes < need)
            return KDA_ERR_WORKSPACE_TOO_SMALL;
    }
    if (N == 0)
        return KDA_OK;
    // one workgroup per (slot, head) on a 1-D grid
    if (dt == KDA_BF16 && n_slots * (int64_t)H > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    if (!tensors_aligned({q, k, v, g, gate, out, init_state, final_state, snapshots}) ||
        !aligned_to(beta, elem_bytes(dt)) || !aligned_to(cu_seqlens, 4) ||
        !aligned_to(workspace, kWorkspaceAlign))
        return KDA_ERR_MISALIGNED;
    const int interval = snapshots ? snapshot_interval : 0;
    if (noalloc && dt == KDA_BF16 && need > 0) {
        const hipError_t e = scratch_address(&workspace);
        if (e != hipSuccess)
            return KDA_ERR_HIP;
    }
    if (dt == KDA_F32)
        return from_hip(kda::launch_chunk_f32(
            (const float *)q, (const float *)k, (const float *)v, (const float *)g,
            (const float *)beta, (const float *)gate, init_state, (float *)out, final_state,
            snapshots, interval, cu_seqlens, N, T, H, scale, prologue, stream));
    return from_hip(kda::launch_chunk_bf16(
        (const kda::bf16 *)q, (const kda::bf16 *)k, (const kda::bf16 *)v, (const kda::bf16 *)g,
        (const kda::bf16 *)beta, (const kda::bf16 *)gate, init_state, (kda::bf16 *)out,
        final_state, snapshots, interval, cu_seqlens, N, T, H, n_slots, scale, prologue,
        workspace, stream, pair, !noalloc));
}

}  // namespace

extern "C" {

kda_status kda_chunk_fwd_ex(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const void *gate, const float *init_state,
                            void *out, float *final_state, float *snapshots,
                            int snapshot_interval, const int32_t *cu_seqlens, int B, int T,
                            int N, int H, int dk, int dv, int chunk, float scale, kda_dtype dt,
                            unsigned flags, void *workspace, size_t workspace_bytes,
                            hipStream_t stream)
{
    return chunk_fwd(q, k, v, g, beta, gate, init_state, out, final_state, snapshots,
                     snapshot_interval, cu_seqlens, B, T, N, H, dk, dv, chunk, scale, dt, flags,
                     workspace, workspace_bytes, stream, false);
}

kda_status kda_chunk_fwd_noalloc(const void *q, const void *k, const void *v, const void *g,
                                 const void *beta, const void *gate, const float *init_state,
                                 void *out, float *final_state, const int32_t *cu_seqlens, int B,
                                 int T, int N, int H, int dk, int dv, int chunk, float scale,
                                 kda_dtype dt, hipStream_t stream)
{
    return chunk_fwd(q, k, v, g, beta, gate, init_state, out, final_state, nullptr, 0,
                     cu_seqlens, B, T, N, H, dk, dv, chunk, scale, dt, 0u, nullptr, 0, stream,
                     true);
}

kda_status kda_chunk_fwd_snapshots(const void *q, const void *k, const void *v, const void *g,
                                   const void *beta, const void *gate, const float *init_state,
                                   void *out, float *final_state, float *snapshots,
                                   int snapshot_interval, const int32_t *cu_seqlens, int B,
                                   int T, int N, int H, int dk, int dv, int chunk, float scale,
                                   kda_dtype dt, void *workspace, size_t workspace_bytes,
                                   hipStream_t stream)
{
    return kda_chunk_fwd_ex(q, k, v, g, beta, gate, init_state, out, final_state, snapshots,
                            snapshot_interval, cu_seqlens, B, T, N, H, dk, dv, chunk, scale, dt,
                            0u, workspace, workspace_bytes, stream);
}

kda_status kda_chunk_fwd(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, const float *init_state,
                         void *out, float *final_state, const int32_t *cu_seqlens, int B, int T,
                         int N, int H, int dk, int dv, int chunk, float scale, kda_dtype dt,
                         void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    return kda_chunk_fwd_ex(q, k, v, g, beta, gate, init_state, out, final_state, nullptr, 0,
                            cu_seqlens, B, T, N, H, dk, dv, chunk, scale, dt, 0u, workspace,
                            workspace_bytes, stream);
}

kda_status kda_decode_step_ex(const void *q, const void *k, const void *v, const void *g,
                              const void *beta, const void *gate, float *state, void *out, int N,
                              int H, int dk, int dv, float scale, kda_dtype dt, unsigned prologue,
                              hipStream_t stream)
{
    if (!valid_dtype(dt))
        return KDA_ERR_BAD_DTYPE;
    if (!decode_supported(dt, dk, dv) || (prologue & ~kProAll) != 0)
        return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H < 1)
        return KDA_ERR_BAD_SHAPE;
    if ((int64_t)N * H > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    if (N == 0)
        return KDA_OK;
    if (!q || !k || !v || !g || !beta || !gate || !state || !out)
        return KDA_ERR_NULL_POINTER;
    if (!tensors_aligned({q, k, v, g, gate, state, out}) || !aligned_to(beta, elem_bytes(dt)))
        return KDA_ERR_MISALIGNED;
    return from_hip(kda::launch_decode(q, k, v, g, beta, gate, state, out, nullptr, N, 1, H, dk,
                                       dv, scale, dt == KDA_BF16, prologue, 1, stream));
}

kda_status kda_decode_verify(const void *q, const void *k, const void *v, const void *g,
                             const void *beta, const void *gate, const float *state, void *out,
                             float *u_out, int N, int K, int H, int dk, int dv, float scale,
                             kda_dtype dt, unsigned prologue, hipStream_t stream)
{
    if (!valid_dtype(dt))
        return KDA_ERR_BAD_DTYPE;
    if (!decode_supported(dt, dk, dv) || (prologue & ~kProAll) != 0)
        return KDA_ERR_UNSUPPORTED;
    if (N < 0 || K < 1 || H < 1)
        return KDA_ERR_BAD_SHAPE;
    if ((int64_t)N * H > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    if (N == 0)
        return KDA_OK;
    if (!q || !k || !v || !g || !beta || !gate || !state || !out)
        return KDA_ERR_NULL_POINTER;
    if (!tensors_aligned({q, k, v, g, gate, state, out, u_out}) ||
        !aligned_to(beta, elem_bytes(dt)))
        return KDA_ERR_MISALIGNED;
    // the state is only read (write_state = 0)
    return from_hip(kda::launch_decode(q, k, v, g, beta, gate, const_cast<float *>(state), out,
                                       u_out, N, K, H, dk, dv, scale, dt == KDA_BF16, prologue, 0,
                                       stream));
}

kda_status kda_decode_commit(const void *k, const void *g, const float *u,
                             const int32_t *accepted, float *state, int N, int K, int H, int dk,
                             int dv, kda_dtype dt, unsigned prologue, hipStream_t stream)
{
    if (!valid_dtype(dt))
        return KDA_ERR_BAD_DTYPE;
    if (!decode_supported(dt, dk, dv) || (prologue & ~kProAll) != 0)
        return KDA_ERR_UNSUPPORTED;
    if (N < 0 || K < 1 || H < 1)
        return KDA_ERR_BAD_SHAPE;
    if ((int64_t)N * H > INT32_MAX)
        return KDA_ERR_UNSUPPORTED;
    if (N == 0)
        return KDA_OK;
    if (!k || !g || !u || !accepted || !state)
        return KDA_ERR_NULL_POINTER;
    if (!tensors_aligned({k, g, u, state}) || !aligned_to(accepted, 4))
        return KDA_ERR_MISALIGNED;
    return from_hip(kda::launch_commit(k, g, u, accepted, state, N, K, H, dk, dv,
                                       dt == KDA_BF16, prologue, stream));
}

int kda_chunk_bwd_supported(kda_dtype dt, int dk, int dv, int chunk)
{
    return bwd_supported(dt, dk, dv, chunk) ? 1 : 0;
}

size_t kda_chunk_bwd_workspace_bytes(int B, int T, int N, int H, int dk, int dv, int chunk,
                                     kda_dtype dt, int varlen)
{
    if (!valid_dtype(dt) || !bwd_supported(dt, dk, dv, chunk))
        return (size_t)-1;
    if (B < 1 || T < 0 || N < 0 || H < 1 || (varlen && B != 1) || (!varlen && N != B))
        return (size_t)-1;
    const size_t units = (size_t)chunk_slots(B, T, N, chunk, varlen) * (size_t)H;
    if (dt == KDA_F32)   // one fp32 dk x dv entry state per (chunk slot, head)
        return units * (size_t)dk * (size_t)dv * sizeof(float);
    return 2 * units * kda::kChunkRecBytes;   // forward and backward records
}

kda_status kda_chunk_bwd_ex(const void *q, const void *k, const void *v, const void *g,
                            const void *beta, const void *gate, const float *init_state,
                            const void *grad_out, const float *grad_final_state, void *grad_q,
                            void *grad_k, void *grad_v, void *grad_g, void *grad_beta,
                            void *grad_gate, float *grad_init_state, const int32_t *cu_seqlens,
                            int B, int T, int N, int H, int dk, int dv, int chunk, float scale,
                            kda_dtype dt, void *fwd_records, size_t fwd_records_bytes,
                            void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    if (!valid_dtype(dt))
        return KDA_ERR_BAD_DTYPE;
    if (!bwd_supported(dt, dk, dv, chunk))
        return KDA_ERR_UNSUPPORTED;
    if (fwd_records && dt != KDA_BF16)
        return KDA_ERR_UNSUPPORTED;
    const int varlen = cu_seqlens != nullptr;
    if (B < 1 || T < 0 || N < 0 || H < 1)
        return KDA_ERR_BAD_SHAPE;
    if (varlen ? B != 1 : N != B)
        return KDA_ERR_BAD_SHAPE;
    const bool has_tokens = (int64_t)B * T > 0;
    if (has_tokens && (!q || !k || !v || !g || !beta || !gate || !grad_out || !grad_q ||
                       !grad_k || !grad_v || !grad_g || !grad_beta || !grad_gate))
        return KDA_ERR_NULL_POINTER;
    size_t need = kda_chunk_bwd_workspace_bytes(B, T, N, H, dk, dv, chunk, dt, varlen);
    if (fwd_records) {
        // the forward's per-chunk records stand in for the first of the two
        // record arrays
        const size_t rec = kda_chunk_fwd_records_bytes(B, T, N, H, dk, dv, chunk, dt, varlen);
        if (fwd_records_bytes < rec)
            return KDA_ERR_WORKSPACE_TOO_SMALL;
        need -= rec;
    }
    if (need > 0 && !workspace)
        return KDA_ERR_NULL_POINTER;
    if (workspace_bytes < need)
        return KDA_ERR_WORKSPACE_TOO_SMALL;
    if (N == 0)
        return KDA_OK;
    // 1-D grids: one workgroup per (sequence, head) or per (chunk slot, head)
    if ((int64_t)N * H > INT32_MAX ||
        (dt == KDA_BF16 && chunk_slots(B, T, N, chunk, varlen) * (int64_t)H > INT32_MAX))
        return KDA_ERR_UNSUPPORTED;
    if (!tensors_aligned({q, k, v, g, gate, init_state, grad_out, grad_final_state, grad_q,
                          grad_k, grad_v, grad_g, grad_gate, grad_init_state}) ||
        !aligned_to(beta, elem_bytes(dt)) || !aligned_to(grad_beta, elem_bytes(dt)) ||
        !aligned_to(cu_seqlens, 4) || !aligned_to(fwd_records, kWorkspaceAlign) ||
        !aligned_to(workspace, kWorkspaceAlign))
        return KDA_ERR_MISALIGNED;
    if (dt == KDA_BF16)
        return from_hip(kda::launch_chunk_bwd_bf16(
            (const kda::bf16 *)q, (const kda::bf16 *)k, (const kda::bf16 *)v,
            (const kda::bf16 *)g, (const kda::bf16 *)beta, (const kda::bf16 *)gate, init_state,
            (const kda::bf16 *)grad_out, grad_final_state, (kda::bf16 *)grad_q,
            (kda::bf16 *)grad_k, (kda::bf16 *)grad_v, (kda::bf16 *)grad_g,
            (kda::bf16 *)grad_beta, (kda::bf16 *)grad_gate, grad_init_state, cu_seqlens, N, T,
            H, chunk_slots(B, T, N, chunk, varlen), scale, fwd_records, workspace, stream));
    return from_hip(kda::launch_chunk_bwd_f32(
        (const float *)q, (const float *)k, (const float *)v, (const float *)g,
        (const float *)beta, (const float *)gate, init_state, (const float *)grad_out,
        grad_final_state, (float *)grad_q, (float *)grad_k, (float *)grad_v, (float *)grad_g,
        (float *)grad_beta, (float *)grad_gate, grad_init_state, cu_seqlens, N, T, H, scale,
        (float *)workspace, stream));
}

kda_status kda_chunk_bwd(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, const float *init_state,
                         const void *grad_out, const float *grad_final_state, void *grad_q,
                         void *grad_k, void *grad_v, void *grad_g, void *grad_beta,
                         void *grad_gate, float *grad_init_state, const int32_t *cu_seqlens,
                         int B, int T, int N, int H, int dk, int dv, int chunk, float scale,
                         kda_dtype dt, void *workspace, size_t workspace_bytes,
                         hipStream_t stream)
{
    return kda_chunk_bwd_ex(q, k, v, g, beta, gate, init_state, grad_out, grad_final_state,
                            grad_q, grad_k, grad_v, grad_g, grad_beta, grad_gate, grad_init_state,
                            cu_seqlens, B, T, N, H, dk, dv, chunk, scale, dt, nullptr, 0,
                            workspace, workspace_bytes, stream);
}

kda_status kda_decode_step(const void *q, const void *k, const void *v, const void *g,
                           const void *beta, const void *gate, float *state, void *out, int N,
                           int H, int dk, int dv, float scale, kda_dtype dt, hipStream_t stream)
{
    return kda_decode_step_ex(q, k, v, g, beta, gate, state, out, N, H, dk, dv, scale, dt, 0u,
                              stream);
}

}  // extern "C"
