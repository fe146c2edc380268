// kda_internal.h -- shared definitions of the gfx950 KDA kernels (not part of
// the public ABI; see include/kda.h for that).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

namespace kda {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16 chunk
// Geometry of the bf16 chunk path: 64-token chunks made of four 16-token
// subtiles, dk = dv = 128, value channels split into 16-wide blocks that run
// as independent recurrences (columns of the state never mix).
constexpr int kChunk = 64;
constexpr int kSub = 16;
constexpr int kDK = 128;
constexpr int kDV = 128;
constexpr int kVBlock = 16;
constexpr int kNumVBlocks = kDV / kVBlock;

// Per-(chunk slot, head) record written by the prep kernel and read by the
// chain kernel.  With L = K'^T W (dk x dk), Bm = K'^T U~ (dk x dv),
// Q^ = Q~ - P W (chunk x dk) and O0 = P U~ (chunk x dv), one chunk maps the
// entry state S to
//     S_next = diag(dec) S + Bm - L S,        O = Q^ S + O0.
// Matrices the chain multiplies are stored as ready-to-load MFMA operand
// fragments of v_mfma_f32_16x16x32_bf16 (64 lanes x 8 bf16 = 1 KiB, lane l at
// byte 16 l) whose k index follows "perm": within a 32-wide k-step ks, lane
// group b = lane / 16 and element e (0..7) stand for row
// 32 ks + 16 (e / 4) + 4 b + (e % 4), which is exactly how the chain holds the
// state in its accumulators.  Additive terms are stored in accumulator order.
//   LN  : -L, 8 dk row tiles x 4 dk k-steps                      (32 KiB)
//   QH  : Q^, 4 chunk row tiles x 4 dk k-steps                   (16 KiB)
//   BM  : Bm per 16-wide value block, [block][wave w][lane][8]:
//         elements 0..3 -> rows 32 w + 4 b + i, 4..7 -> rows 32 w + 16 + 4 b + i,
//         column 16 block + lane % 16                              (32 KiB)
//   O0  : O0 per value block, [block][row tile pair tp][lane][8]: elements
//         4 s .. 4 s + 3 -> row 16 (2 tp + s) + lane % 16, columns 16 block + 4 b .. + 3
//                                                                  (16 KiB)
//   DEC : exp(G_end) per key channel, fp32                        (512 B)
//   SB  : the state on entry to the chunk, per value block, as the 4 k-step
//         B fragments (bf16, perm order) the output product reads  (32 KiB)
// LN, QH, BM, O0 and DEC are written by the prep kernel, SB by the chain.
constexpr size_t kFragBytes = 1024;
constexpr size_t kOffLN = 0;
constexpr size_t kOffQH = kOffLN + 32 * kFragBytes;
constexpr size_t kOffBM = kOffQH + 16 * kFragBytes;
constexpr size_t kOffO0 = kOffBM + kNumVBlocks * 4096;
constexpr size_t kOffDEC = kOffO0 + kNumVBlocks * 2048;
constexpr size_t kOffSB = kOffDEC + kDK * sizeof(float);
constexpr size_t kRecBytes = kOffSB + kNumVBlocks * 4 * kFragBytes;
static_assert(kRecBytes % 256 == 0, "records stay 256-byte aligned");

// Pair record: two consecutive chunks of a sequence whose maps are composed
// into one step of the chain.  With M = diag(dec) - L the map of one chunk,
// chunks 0 and 1 of a pair give S'' = M1 M0 S + M1 Bm0 + Bm1, i.e.
//     dec01 = dec0 dec1,   L01 = L1 D0 + M1 L0,   Bm01 = Bm1 + M1 Bm0,
// and the outputs of chunk 1 from the pair's entry state S are
//     O1 = Q^1 (M0 S + Bm0) + O0_1 = Q^1' S + O0_1',
//     Q^1' = Q^1 D0 - Q^1 L0,   O0_1' = O0_1 + Q^1 Bm0.
// (D = diag(dec); the decays enter the products only as D0 scaling columns
// in fp32 and inside M1, which multiplies L0 and Bm0, so no decay is rounded
// to bf16 on its own.)  The first kRecBytes bytes have the layout of a chunk record (LN, BM, DEC:
// the composed map; QH, O0: chunk 0's readout; SB: the state on entry to the
// pair); after them:
//   QH1 : Q^1', QH layout                                          (16 KiB)
//   O01 : O0_1', O0 layout                                         (16 KiB)
// A sequence's last pair may hold one chunk; it then carries that chunk's
// own map and readout, and QH1 / O01 are not used.
constexpr int kPairTokens = 2 * kChunk;
constexpr size_t kOffQH1 = kRecBytes;
constexpr size_t kOffO01 = kOffQH1 + 16 * kFragBytes;
constexpr size_t kPairRecBytes = kOffO01 + kNumVBlocks * 2048;
static_assert(kPairRecBytes % 256 == 0, "pair records stay 256-byte aligned");

// Per-chunk records (kept for the backward, or for snapshots inside a pair)
// add the chunk's intra-chunk factors after the first kRecBytes bytes, for
// the chunk-level gradient kernel:
//   XW : W = T diag(beta) K e^G as row fragments: fragment (token row tile t,
//        dk k-step ks) at (4 t + ks) KiB, lane (b, m) holding row 16 t + m,
//        dk 32 ks + 16 (e / 4) + 4 b + e % 4 (perm order)              (16 KiB)
//   XU : U~ = T diag(beta) V, the same layout over dv                  (16 KiB)
//   XT : T^T, bf16 [64][64] row-major (XT[r][s] = T[s][r])             (8 KiB)
//   XP : P^T, bf16 [64][64] row-major, P = scale * lower_incl(Q e^G (K e^-G)^T)
//                                                                       (8 KiB)
constexpr size_t kOffXW = kRecBytes;
constexpr size_t kOffXU = kOffXW + 16 * kFragBytes;
constexpr size_t kOffXT = kOffXU + 16 * kFragBytes;
constexpr size_t kOffXP = kOffXT + (size_t)kChunk * kChunk * 2;
constexpr size_t kChunkRecBytes = kOffXP + (size_t)kChunk * kChunk * 2;
static_assert(kChunkRecBytes % 256 == 0, "chunk records stay 256-byte aligned");

// Global-memory pointers whose address space is explicit, so the compiler
// emits global (not flat) memory instructions for them.
typedef __attribute__((address_space(1))) uint8_t gbyte;

// A wave-uniform pointer made visibly uniform (scalar registers), so that
// memory accesses through it take the scalar-base + 32-bit vector-offset form
// instead of a 64-bit address per lane, which halves the address traffic of
// every vector memory instruction.
__device__ __forceinline__ const gbyte *uniform_gptr(const void *p)
{
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const gbyte *>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ gbyte *uniform_gptr(void *p)
{
    return const_cast<gbyte *>(uniform_gptr(static_cast<const void *>(p)));
}

// Load / store a T at byte offset off from a global base pointer.
template <typename T> __device__ __forceinline__ T gload(const gbyte *base, uint32_t off)
{
    return *reinterpret_cast<const __attribute__((address_space(1))) T *>(base + off);
}
template <typename T> __device__ __forceinline__ void gstore(gbyte *base, uint32_t off, const T &v)
{
    *reinterpret_cast<__attribute__((address_space(1))) T *>(base + off) = v;
}

// Row of the k-step-local permutation described above.
__host__ __device__ constexpr int perm_row(int ks, int b, int e)
{
    return 32 * ks + 16 * (e >> 2) + 4 * b + (e & 3);
}

__device__ __forceinline__ f32x4 mfma16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 lds8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

// 8 bf16 in perm order from a row with the k index contiguous:
// elements 0..3 <- p[32 ks + 4 b + 0..3], 4..7 <- p[32 ks + 16 + 4 b + 0..3]
__device__ __forceinline__ bf16x8 perm8(const bf16 *row, int ks, int b)
{
    const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(row + 32 * ks + 4 * b);
    const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(row + 32 * ks + 16 + 4 * b);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// accumulator tiles (2 ks, 2 ks + 1) -> one perm-order fragment
__device__ __forceinline__ bf16x8 acc_to_frag(const f32x4 &lo, const f32x4 &hi)
{
    return bf16x8{(bf16)lo[0], (bf16)lo[1], (bf16)lo[2], (bf16)lo[3],
                  (bf16)hi[0], (bf16)hi[1], (bf16)hi[2], (bf16)hi[3]};
}

// D += A B with a 16-wide k: lane (b, m) gives A[m][4 b + e] and B[4 b + e][m]
// (e = 0..3).  Issued as the 16x16x32 product with elements 4..7 of both
// operands zero (k = 8 b + e then stands for 4 b + e on both sides), so that
// every bf16 matrix instruction of the kernel has one shape: a 16x16x16
// accumulating directly onto a chain of 16x16x32 products has been seen to
// read part of its accumulator input stale on gfx950.
__device__ __forceinline__ f32x4 mfma16k16(const bf16x4 &a, const bf16x4 &b, const f32x4 &c)
{
    const bf16 z = (bf16)0.f;
    return mfma16(bf16x8{a[0], a[1], a[2], a[3], z, z, z, z},
                  bf16x8{b[0], b[1], b[2], b[3], z, z, z, z}, c);
}

// fp32 16x16x4: lane l gives A[l % 16][l / 16] and B[l / 16][l % 16]
__device__ __forceinline__ f32x4 mfma4_f32(float a, float b, const f32x4 &c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// DPP lane move (as int bits) with every lane active; lanes whose source is
// out of range (bound_ctrl) or whose row is masked off read 0
template <int kCtrl, int kRowMask, bool kBound>
__device__ __forceinline__ float dpp_add_src(float x)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), kCtrl, kRowMask, 0xf, kBound));
}

// inclusive prefix sum over each 16-lane row of a wave (row_shr 1, 2, 4, 8;
// lanes whose source falls outside the row add 0)
__device__ __forceinline__ float row_inclusive_sum(float x)
{
    x += dpp_add_src<0x111, 0xf, true>(x);
    x += dpp_add_src<0x112, 0xf, true>(x);
    x += dpp_add_src<0x114, 0xf, true>(x);
    x += dpp_add_src<0x118, 0xf, true>(x);
    return x;
}

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }

__device__ __forceinline__ float sigmoidf_(float x) { return 1.0f / (1.0f + __expf(-x)); }

// ------------------------------------------------------------- prologue
// Optional input maps applied inside the kernels (same bits as KDA_PRO_* in
// kda.h): q and k L2-normalised over dk per (token, head) with the epsilon
// inside the square root, beta = sigmoid(logit), g = max(-5, -softplus(x)).
constexpr unsigned kProQK = 1u, kProBeta = 2u, kProG = 4u;
constexpr float kNormEps = 1e-6f;

__device__ __forceinline__ float log_decay_from(float x)
{
    const float sp = fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)));   // softplus(x)
    return fmaxf(-5.f, -sp);
}

// Sequence bounds and first chunk slot of sequence n.  Without cu_seqlens the
// B sequences have length T and slot = n * ceil(T / chunk) + j.  With
// cu_seqlens, slot(n, j) = floor(cu[n] / chunk) + n + j, an injective map
// into [0, floor(T / chunk) + N) that needs no prefix scan.
struct SeqInfo {
    int64_t bos;
    int64_t len;
    int64_t slot0;
};

__device__ __forceinline__ SeqInfo seq_info(const int32_t *cu, int n, int T, int chunk)
{
    SeqInfo s;
    if (cu) {
        int64_t a = cu[n], b = cu[n + 1];
        s.bos = a;
        s.len = b - a;
        s.slot0 = a / chunk + n;
    } else {
        s.bos = (int64_t)n * T;
        s.len = T;
        s.slot0 = (int64_t)n * ((T + chunk - 1) / chunk);
    }
    return s;
}

// Slot of kStep tokens (a chunk, or a pair of chunks) -> (sequence, step
// index).  Returns false for an unused slot.
template <int kStep>
__device__ __forceinline__ bool slot_to_step(const int32_t *cu, int N, int T, int64_t slot, int &n,
                                             int64_t &j)
{
    if (cu) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {                       // largest n with cu[n]/C + n <= slot
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)cu[mid] / kStep + mid <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        n = lo;
        j = slot - ((int64_t)cu[n] / kStep + n);
        return (int64_t)cu[n + 1] - cu[n] > j * kStep;
    }
    const int64_t nck = (T + kStep - 1) / kStep;
    n = (int)(slot / nck);
    j = slot % nck;
    return n < N;
}

// Chunk slot -> (sequence, chunk index).  Returns false for an unused slot.
__device__ __forceinline__ bool slot_to_chunk(const int32_t *cu, int N, int T, int64_t slot,
                                              int &n, int64_t &j)
{
    return slot_to_step<kChunk>(cu, N, T, slot, n, j);
}


// First snapshot slot of sequence n for snapshots every `interval` tokens
// (a multiple of the chunk length).  Snapshot m = 1 .. floor(len / interval)
// of sequence n, the state after its first m * interval tokens, goes to slot
// snap_slot0(n) + m - 1.  Without cu_seqlens that is n * floor(T / interval)
// + m - 1; with cu_seqlens floor(cu[n] / interval) + n + m - 1, injective into
// [0, floor(T / interval) + N) for the same reason as the chunk slots.
__device__ __forceinline__ int64_t snap_slot0(const int32_t *cu, int n, int T, int interval)
{
    return cu ? (int64_t)cu[n] / interval + n : (int64_t)n * (T / interval);
}

// ------------------------------------------------------------- launchers
// All return hipSuccess or the launch error.
// Decode step (K = 1, write_state = 1, u_out NULL) or verification of K
// tokens (write_state = 0, u_out = the corrections for launch_commit).
hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, float *state, void *out,
                         float *u_out, int N, int K, int H, int dk, int dv, float scale,
                         int is_bf16, unsigned pro, int write_state, hipStream_t stream);

hipError_t launch_commit(const void *k, const void *g, const float *u, const int32_t *accepted,
                         float *state, int N, int K, int H, int dk, int dv, int is_bf16,
                         unsigned pro, hipStream_t stream);

// snaps / snap_interval: state snapshots (see snap_slot0); NULL / 0 for none.
hipError_t launch_chunk_f32(const float *q, const float *k, const float *v, const float *g,
                            const float *beta, const float *gate, const float *init,
                            float *out, float *final_state, float *snaps, int snap_interval,
                            const int32_t *cu, int N, int T, int H, float scale, unsigned pro,
                            hipStream_t stream);

// Chunkwise backward, fp32, dk = dv = 16, 16-token chunks; ws holds one
// 16 x 16 fp32 entry state per (chunk slot, head).
hipError_t launch_chunk_bwd_f32(const float *q, const float *k, const float *v, const float *g,
                                const float *beta, const float *gate, const float *init,
                                const float *dout, const float *dfinal, float *dq, float *dk,
                                float *dv, float *dg, float *dbeta, float *dgate, float *dinit,
                                const int32_t *cu, int N, int T, int H, float scale, float *ws,
                                hipStream_t stream);

// allow_aux = false keeps every kernel on `stream` (no auxiliary stream is
// created or used, whatever the sequence length).  pair = true composes
// consecutive chunks into pair records (n_slots then counts pair slots:
// B ceil(T / 128), or floor(T / 128) + N with cu_seqlens); snapshots then
// need an interval that is a multiple of kPairTokens.
hipError_t launch_chunk_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                             const bf16 *beta, const bf16 *gate, const float *init, bf16 *out,
                             float *final_state, float *snaps, int snap_interval,
                             const int32_t *cu, int N, int T, int H, int64_t n_slots,
                             float scale, unsigned pro, void *workspace, hipStream_t stream,
                             bool pair, bool allow_aux = true);

// Chunkwise backward, bf16, dk = dv = 128, 64-token chunks; the workspace
// holds two record arrays of n_slots * H records each (forward, backward), or
// only the backward one when fwd_records holds a forward call's records.
hipError_t launch_chunk_bwd_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                                 const bf16 *beta, const bf16 *gate, const float *init,
                                 const bf16 *dout, const float *dfinal, bf16 *dq, bf16 *dk,
                                 bf16 *dv, bf16 *dg, bf16 *dbeta, bf16 *dgate, float *dinit,
                                 const int32_t *cu, int N, int T, int H, int64_t n_slots,
                                 float scale, void *fwd_records, void *workspace,
                                 hipStream_t stream);

// Devices with per-device library state (kernel attributes, the second
// stream of the long-sequence schedule, the static workspace).
constexpr int kMaxDevices = 64;

// Runs set() once per device, with that device current, and returns its
// result to every call on that device (kSite tells the callers apart).  For
// kernel attributes such as the dynamic LDS limit, which are set per device.
template <int kSite> inline hipError_t once_per_device(hipError_t (*set)())
{
    static std::once_flag flag[kMaxDevices];
    static hipError_t err[kMaxDevices];
    int dev = 0;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::call_once(flag[dev], [&] { err[dev] = set(); });
    return err[dev];
}

// Backward records: for chunk j of a sequence with nch chunks, record
// slot0 + nch - 1 - j of ws_b gets LN = -L^T, BM = Q^^T dO (dO = dY sigmoid(Z))
// and DEC of the forward record of chunk j in ws_f, so that the chain walks
// the chunks last to first.
hipError_t launch_bwd_prep_bf16(const bf16 *gate, const bf16 *dout, const int32_t *cu, int N,
                                int T, int H, int64_t n_slots, const uint8_t *ws_f,
                                uint8_t *ws_b, hipStream_t stream);

// Per-chunk gradients from the forward records (Q^, O0, the entry state SB and
// the extension XW, XU, XT, XP) and the exit state gradients (SB of the
// reversed records of ws_b); writes no record.
hipError_t launch_grad_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                            const bf16 *beta, const bf16 *gate, const bf16 *dout, bf16 *dq,
                            bf16 *dk, bf16 *dv, bf16 *dg, bf16 *dbeta, bf16 *dgate,
                            const int32_t *cu, int N, int T, int H, int64_t n_slots, float scale,
                            uint8_t *ws_f, const uint8_t *ws_b, hipStream_t stream);

}  // namespace kda
