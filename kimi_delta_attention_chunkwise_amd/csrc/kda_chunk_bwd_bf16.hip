// kda_chunk_bwd_bf16.hip -- chunkwise KDA backward for bf16 inputs,
// dk = dv = 128, 64-token chunks, fp32 state and gradients of the state.
//
// Source: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
// section 1 row Q07 (the chunkwise-parallel form serves training as well as
// prefill) and row Q06 (g >= -5 bounds the decay inside a 16-token subtile).
//
// The forward maps the state on entry to chunk j to the next one with
//     S_{j+1} = (diag(dec) - L) S_j + Bm,      O_j = Q^ S_j + O0
// (the records of the forward prep).  Its adjoint walks the chunks backward:
//     dS_j = (diag(dec) - L^T) dS_{j+1} + Q^^T dO_j,    dO = dY sigmoid(Z),
// which is the same recurrence with L^T for L and Q^^T dO for Bm.  So:
//   1. forward prep + chain: every chunk's entry state S_j (record SB);
//   2. backward records with -L^T, Q^^T dO and dec, stored in reverse chunk
//      order: written by the forward prep itself when the backward runs its
//      own forward, or by the backward prep kernel (here) from the records of
//      an earlier forward call, so that
//   3. the same chain kernel, started from dS_final, yields dS_{j+1} for
//      every chunk (record SB) and dS_0 (in one launch with step 1's chain
//      when the backward runs its own forward);
//   4. gradient kernel (here): one workgroup per (chunk, head) computes the
//      chunk's gradients at chunk level from the forward record (Q^, O0, the
//      entry state S and the per-chunk extension W, U~, T^T, P^T written by
//      the prep) and dS' = dS_{j+1}; no pass over the chunk is serial.
//
// Algebra of one 64-token chunk with entry state S (r, s its rows; G the
// cumulative log-decay from the chunk start including the row; Ge = G of the
// last row; B_I = G before 16-token subtile I, B_0 = 0):
//   Qs = scale Q e^G, Ks = K e^G, Kp = K e^{Ge-G};  M = strict_lower([k_r e^{G_r-G_s} k_s]),
//   A = diag(beta) M, P = scale lower_incl([q_r e^{G_r-G_s} k_s]), T = (I + A)^-1,
//   W = T diag(beta) Ks, U~ = T diag(beta) V, U = U~ - W S, O = Q^ S + O0 = Qs S + P U,
//   S' = diag(e^Ge) S + Kp^T U.
// Backward, given dS' and dO = dY sigmoid(Z):
//   dU = Kp dS' + P^T dO,  dKp = U dS'^T, dQs = dO S^T, dW = -dU S^T,
//   dP = lower_incl(dO U^T),  dX = T^T dW, dY~ = T^T dU,
//   dA = -T^T dT T^T = strict_lower(-dX W^T - dY~ U~^T)
//        (dT = dW (diag(beta) Ks)^T + dU (diag(beta) V)^T and T X = W, T Y = U~),
//   dKs = diag(beta) dX, dV = diag(beta) dY~, dbeta = rowsum(dX Ks + dY~ V + dA M).
// The products with the 16 x 16 blocks of A and P carry the decay with
// references at subtile starts: with Kr_I = K_I e^{G - B_I}, Qr_I = scale Q_I e^{G - B_I}
// and Kc_J^(I) = K_J e^{B_I - G} for block (I, J), J <= I,
//   Z_I = sum_J dA_IJ Kc_J^(I),  dKr_I = diag(beta) Z_I,  dQr_I = sum_J dP_IJ Kc_J^(I),
//   dKc_J = sum_{I >= J} (diag(beta) dA_IJ)^T Kr_I^(J) + dP_IJ^T Qr_I^(J)
//   (row factors K_I e^{G - B_J}, scale Q_I e^{G - B_J}: references B_J), and
//   dM's rowsum term of dbeta is rowsum(Kr Z);
//   dQ = scale (e^G dQs + e^{G-B} dQr), dK = e^G dKs + e^{G-B} dKr + e^{B-G} dKc + e^{Ge-G} dKp,
//   dG = dQs Qs + dQr Qr + dKs Ks + dKr Kr - dKc Kc - dKp Kp,
//   dGe = colsum(dKp Kp) + e^Ge rowsum(dS' S),  dg_u = sum_{r >= u} dG_r + dGe.
// The references cancel inside M and P, so they carry no gradient.  Every
// factor stays in range because g >= -5 and a subtile is 16 tokens: e^{G - B}
// lies in [e^-80, 1] on its own subtile, e^{B - G} in [1, e^80], and every
// factor between different subtiles is at most 1.
#include "kda_internal.h"

#include <mutex>

namespace kda {

namespace {

// ------------------------------------------------------------ backward prep
constexpr int kBpThreads = 512;

// column of token r in row c of OT (see the dO staging below)
__device__ __forceinline__ int ot_col(int c, int r) { return 8 * ((r >> 3) ^ ((c >> 4) & 7)) + (r & 7); }

struct BwdPrepSmem {
    bf16 L[kDK][kDK + 8];           // -L, row-major
    bf16 QT[kDK][kChunk + 8];       // Q^^T  [dk][token]
    bf16 OT[kDV][kChunk + 8];       // dO^T  [dv][token]
};

__global__ __launch_bounds__(kBpThreads) void kda_bwd_prep_bf16_kernel(
    const bf16 *__restrict__ gate, const bf16 *__restrict__ dout, const int32_t *__restrict__ cu,
    int N, int T, int H, const uint8_t *__restrict__ ws_f, uint8_t *__restrict__ ws_b)
{
    extern __shared__ __align__(16) uint8_t smem_raw[];
    BwdPrepSmem &sm = *reinterpret_cast<BwdPrepSmem *>(smem_raw);
    const int64_t slot = (int64_t)blockIdx.x / H;
    const int h = (int)((int64_t)blockIdx.x % H);
    int n;
    int64_t j;
    if (!slot_to_chunk(cu, N, T, slot, n, j))
        return;
    const SeqInfo si = seq_info(cu, n, T, kChunk);
    const int64_t nch = (si.len + kChunk - 1) / kChunk;
    const int64_t tok0 = si.bos + j * kChunk;
    const int len = (int)((si.len - j * kChunk) < kChunk ? (si.len - j * kChunk) : kChunk);
    const uint8_t *rf = ws_f + (slot * H + h) * (int64_t)kChunkRecBytes;
    uint8_t *rb = ws_b + ((si.slot0 + nch - 1 - j) * H + h) * (int64_t)kChunkRecBytes;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 15, b = lane >> 4;

    // -L fragments (row 16 mt + m, perm k order) -> dense rows; 4 lane slots per thread
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int idx = it * kBpThreads + tid;
        const int f = idx >> 6, l = idx & 63;
        const int mt = f >> 2, ks = f & 3, fb = l >> 4, fm = l & 15;
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(rf + kOffLN + f * kFragBytes + l * 16);
        bf16 *row = &sm.L[16 * mt + fm][0];
        *reinterpret_cast<bf16x4 *>(row + 32 * ks + 4 * fb) = bf16x4{x[0], x[1], x[2], x[3]};
        *reinterpret_cast<bf16x4 *>(row + 32 * ks + 16 + 4 * fb) = bf16x4{x[4], x[5], x[6], x[7]};
    }
    // Q^ fragments (token row 16 mt + m, perm dk order) -> Q^^T
#pragma unroll
    for (int it = 0; it < 2; ++it) {
        const int idx = it * kBpThreads + tid;
        const int f = idx >> 6, l = idx & 63;
        const int mt = f >> 2, ks = f & 3, fb = l >> 4, fm = l & 15;
        const bf16x8 x = *reinterpret_cast<const bf16x8 *>(rf + kOffQH + f * kFragBytes + l * 16);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            sm.QT[perm_row(ks, fb, e)][16 * mt + fm] = x[e];
    }
    // dO = dY sigmoid(Z) of token r, channels c0 .. c0 + 15, transposed; zero past
    // the chunk.  OT keeps the 8-token group of row c at group ^ ((c >> 4) & 7)
    // (ot_col): the rows a wave writes at once are 16 apart, which without the
    // permutation would all share one LDS bank.
    {
        const int r = tid >> 3, c0 = 16 * (tid & 7);
        bf16x8 dy[2] = {}, z[2] = {};
        if (r < len) {
            const int64_t off = ((tok0 + r) * H + h) * (int64_t)kDV + c0;
#pragma unroll
            for (int p = 0; p < 2; ++p) {
                dy[p] = *reinterpret_cast<const bf16x8 *>(dout + off + 8 * p);
                z[p] = *reinterpret_cast<const bf16x8 *>(gate + off + 8 * p);
            }
        }
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                sm.OT[c0 + 8 * p + e][ot_col(c0 + 8 * p + e, r)] =
                    (bf16)(r < len ? (float)dy[p][e] * sigmoidf_((float)z[p][e]) : 0.f);
    }
    if (tid < kDK / 4)
        *reinterpret_cast<f32x4 *>(rb + kOffDEC + tid * 16) =
            *reinterpret_cast<const f32x4 *>(rf + kOffDEC + tid * 16);
    __syncthreads();

    // -L^T fragments of row tile w: element e of lane (b, m) = -L[perm_row(ks, b, e)][16 w + m]
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        bf16x8 x;
#pragma unroll
        for (int e = 0; e < 8; ++e)
            x[e] = sm.L[perm_row(ks, b, e)][16 * w + m];
        *reinterpret_cast<bf16x8 *>(rb + kOffLN + (w * 4 + ks) * kFragBytes + lane * 16) = x;
    }
    // Q^^T dO for value block w, in the record's Bm layout: fragment i2 holds row
    // tiles 2 i2 (elements 0..3) and 2 i2 + 1 (elements 4..7)
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
        f32x4 acc[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
            const int t = 2 * i2 + s2;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                a = mfma16(lds8(&sm.QT[16 * t + m][32 * ks + 8 * b]),
                           lds8(&sm.OT[16 * w + m][8 * ((4 * ks + b) ^ w)]), a);
            acc[s2] = a;
        }
        *reinterpret_cast<bf16x8 *>(rb + kOffBM + w * 4096 + i2 * 1024 + lane * 16) =
            acc_to_frag(acc[0], acc[1]);
    }
}

// ------------------------------------------------------------ gradient kernel
constexpr int kGThreads = 512;
constexpr int kGWaves = kGThreads / 64;
constexpr int kXL = kDK + 8;     // bf16 row stride of [64][128] and [128][128] tiles
constexpr int kTL = kChunk + 8;  // bf16 row stride of [64][64] tiles
constexpr int kAL = kChunk + 4;  // fp32 row stride of [64][64] tiles

// Lane kS of the caller's 16-lane row, to every lane of that row (DPP
// row_newbcast: a VALU move, no LDS traffic).
template <int kS>
__device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + kS, 0xf, 0xf, false));
}

__device__ __forceinline__ bf16x4 bf4(const f32x4 &x)
{
    return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// Zero the optimizer cannot see through (an empty asm statement that claims
// to modify it; no instruction).  The LDS base is re-derived from it at the
// top of every phase: the kernel's LDS spans more than the 16-bit offset of
// LDS instructions, and without it the compiler keeps dozens of per-lane LDS
// addresses of later phases live from the first one, which forces spills.
__device__ __forceinline__ uint32_t opaque_zero()
{
    uint32_t z = 0;
    asm volatile("" : "+s"(z));
    return z;
}

// A 16 x 16 tile from the row layout to accumulator order (see the kernel),
// exactly, as its product with the identity: lane (b, m) gives elements
// (token m, channel 4 b + e) and receives (token 4 b + i, channel m).
// The identity's position comes from an opaque copy of the lane index, so
// that transposes in different phases are formed again where they are used
// instead of being merged and held in registers in between.
__device__ __forceinline__ bf16x4 acc_order(const bf16x4 &x, int b, int m)
{
    int mm = m;
    asm volatile("" : "+v"(mm));
    bf16x4 id;
#pragma unroll
    for (int e = 0; e < 4; ++e)
        id[e] = (bf16)(4 * b + e == mm ? 1.f : 0.f);
    return bf4(mfma16k16(x, id, f32x4{0.f, 0.f, 0.f, 0.f}));
}
__device__ __forceinline__ f32x4 acc_order(const f32x4 &x, int b, int m)
{
    int mm = m;
    asm volatile("" : "+v"(mm));
    f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
        d = mfma4_f32(x[kk], 4 * b + kk == mm ? 1.f : 0.f, d);
    return d;
}

__device__ __forceinline__ f32x4 f4(const bf16x4 &x)
{
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
}

// LDS of the gradient kernel, by phase (see the kernel): 153,344 bytes, one
// workgroup per CU.
struct GradSmem {
    union {
        struct {                          // phase 1: the record's Q^ and W fragments
            bf16x8 QH[16][64];
            bf16x8 W[16][64];
        } f;
        struct {                          // phase 2: S and dS' as [dk][dv] tiles
            bf16 Sb[kDK][kXL];
            bf16 dSb[kDK][kXL];
        } s;
        struct {                          // phases 3 to 5
            bf16 DX[kChunk][kXL];         // T^T dW   [token][dk]
            bf16 DY[kChunk][kXL];         // T^T dU   [token][dv]
            float dA[kChunk][kAL];
            float dPT[kChunk][kAL];       // dP^T
        } x;
    } a;
    union {
        struct {                          // phases 1 to 3
            bf16 DO[kChunk][kXL];         // dO = dY sigmoid(Z)   [token][dv]
            bf16 U[kChunk][kXL];          // U = U~ - W S
            bf16 DU[kChunk][kXL];         // dU
        } d;
        float dAbT[kChunk][kAL];          // phases 4, 5: (diag(beta) dA)^T
    } d;
    union {
        bf16 KP[kChunk][kXL];             // K' = K e^{Ge - G} (phase 1)
        float dP[kChunk][kAL];            // phases 2 to 5
    } p;
    union {
        bf16 PT[kChunk][kTL];             // P^T (phase 1)
        bf16 TT[kChunk][kTL];             // T^T (phase 3)
    } t;
    alignas(16) float beta[kChunk];
    alignas(16) float ref[4][kDK];        // G before subtiles 1, 2, 3 (B_1..B_3) and G_end
    alignas(16) float dgeD[kDK];          // e^Ge rowsum(dS' S) per key channel
    alignas(16) float dbp[kGWaves][kChunk];   // per-wave partial sums of dbeta
};
static_assert(sizeof(GradSmem) <= 160 * 1024, "gradient kernel LDS fits one CU");

// G before tile t (B_t; B_0 = 0) of channels c .. c + 3
__device__ __forceinline__ f32x4 ref4(const GradSmem &sm, int t, int c)
{
    return t == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : *reinterpret_cast<const f32x4 *>(&sm.ref[t - 1][c]);
}

// Block (I, J) of a 4 x 4 lower block triangle for wave w; waves 0 and 1 take
// a second one (nb = 1): 0:(0,0) 9:(3,3) / 2:(1,1) 5:(2,2) / 1, 3, 4, 6, 7, 8.
__device__ __forceinline__ void lower_block(int w, int nb, int &I, int &J)
{
    const int blk = w == 0 ? 9 * nb : w == 1 ? 2 + 3 * nb : w == 2 ? 1 : w < 5 ? w : w + 1;
    I = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
    J = blk - (I * (I + 1)) / 2;
}

// One workgroup of 8 waves per (chunk, head).  Two register layouts:
//   row layout: element [t][i] of lane (b, m) is token 16 t + m, channel
//     16 w + 4 b + i -- the accumulator of a product whose MFMA rows are the
//     wave's 16 channels and whose columns are tokens; four consecutive
//     channels of one token, so loads and stores of a row are 8 bytes;
//   accumulator order: element [t][i] is token 16 t + 4 b + i, channel
//     16 w + m -- the operand of a product over tokens (16-wide k).
// Wave w owns value block w (phase 1, dY~) and key block w (phases 2, 3, 5).
__global__ __launch_bounds__(kGThreads) void kda_grad_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, const bf16 *__restrict__ gate,
    const bf16 *__restrict__ dout, bf16 *__restrict__ dq, bf16 *__restrict__ dk,
    bf16 *__restrict__ dv, bf16 *__restrict__ dg, bf16 *__restrict__ dbeta,
    bf16 *__restrict__ dgate, const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    const uint8_t *__restrict__ ws_f, const uint8_t *__restrict__ ws_b)
{
    extern __shared__ __align__(16) uint8_t smem_raw[];
    // re-derived from an opaque zero at the top of every phase (see opaque_zero)
    GradSmem *smp = reinterpret_cast<GradSmem *>(smem_raw);
    const int64_t slot = (int64_t)blockIdx.x / H;
    const int h = (int)((int64_t)blockIdx.x % H);
    int n;
    int64_t j;
    if (!slot_to_chunk(cu, N, T, slot, n, j))
        return;
    const SeqInfo si = seq_info(cu, n, T, kChunk);
    const int64_t nch = (si.len + kChunk - 1) / kChunk;
    const int64_t tok0 = si.bos + j * kChunk;
    const int len = (int)((si.len - j * kChunk) < kChunk ? (si.len - j * kChunk) : kChunk);
    // wave-uniform bases, per-lane 32-bit byte offsets
    const gbyte *rf = uniform_gptr(ws_f + (slot * H + h) * (int64_t)kChunkRecBytes);
    const gbyte *rb = uniform_gptr(ws_b + ((si.slot0 + nch - 1 - j) * H + h) * (int64_t)kChunkRecBytes);
    const int64_t e0 = (tok0 * H + h) * (int64_t)kDK;   // (first token, head h, channel 0)
    const gbyte *gq = uniform_gptr(q + e0), *gk = uniform_gptr(k + e0), *gv_ = uniform_gptr(v + e0);
    const gbyte *gg = uniform_gptr(g + e0), *gz = uniform_gptr(gate + e0);
    const gbyte *gy = uniform_gptr(dout + e0);
    gbyte *oq = uniform_gptr(dq + e0), *ok_ = uniform_gptr(dk + e0), *ov = uniform_gptr(dv + e0);
    gbyte *og_ = uniform_gptr(dg + e0), *oz = uniform_gptr(dgate + e0);
    const uint32_t tstride = (uint32_t)H * kDK * 2;       // bytes from one token to the next

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, b = lane >> 4;
    const int c0 = 16 * w + 4 * b;            // the lane's channels in the row layout
    // byte offset of (token 16 t + m, channel c0) in a [.., H, 128] tensor from
    // the chunk's base; a row past the chunk's end reads its last row (in
    // range), zeroed where used
    auto roff = [&](int t) -> uint32_t {
        const int r = 16 * t + m < len ? 16 * t + m : len - 1;
        return (uint32_t)r * tstride + 2 * c0;
    };

    // ---- phase 0: record operands into LDS, G, K' ----------------------------
    bf16x8 sf[4], df[4];        // S and dS' of value block w as B fragments (perm order)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        sf[ks] = gload<bf16x8>(rf, kOffSB + w * 4096 + ks * 1024 + lane * 16);
        df[ks] = gload<bf16x8>(rb, kOffSB + w * 4096 + ks * 1024 + lane * 16);
    }
    {
        const int r = tid >> 3, c8 = 8 * (tid & 7);
        const bf16x8 q0 = gload<bf16x8>(rf, kOffQH + 16 * tid);
        const bf16x8 q1 = gload<bf16x8>(rf, kOffQH + 16 * (tid + kGThreads));
        const bf16x8 w0 = gload<bf16x8>(rf, kOffXW + 16 * tid);
        const bf16x8 w1 = gload<bf16x8>(rf, kOffXW + 16 * (tid + kGThreads));
        const bf16x8 p8 =
            gload<bf16x8>(rf, kOffXP + (size_t)(r * kChunk + c8) * 2);
        bf16x8 *sq = &smp->a.f.QH[0][0], *sw = &smp->a.f.W[0][0];
        sq[tid] = q0;
        sq[tid + kGThreads] = q1;
        sw[tid] = w0;
        sw[tid + kGThreads] = w1;
        *reinterpret_cast<bf16x8 *>(&smp->t.PT[r][c8]) = p8;
        if (tid < kChunk)
            smp->beta[tid] = tid < len ? (float)beta[(tok0 + tid) * H + h] : 0.f;
    }
    // G (row layout): prefix over the 16 tokens of a tile (DPP), carried over the
    // tiles; G before tiles 1..3 (the references of those subtiles) and G_end
    // go to LDS
    float G[4][4];
    bf16x4 kv[4], qv[4];                      // k and q of the lane's elements (zero past the end)
    {
        bf16x4 gv[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            gv[t] = gload<bf16x4>(gg, roff(t));
            kv[t] = gload<bf16x4>(gk, roff(t));
            qv[t] = gload<bf16x4>(gq, roff(t));
        }
        float carry[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool ok = 16 * t + m < len;
            if (!ok) {
                kv[t] = bf16x4{};
                qv[t] = bf16x4{};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float incl = row_inclusive_sum(ok ? (float)gv[t][i] : 0.f);
                G[t][i] = carry[i] + incl;
                carry[i] += row_bcast<15>(incl);
            }
            if (m == 0)
                *reinterpret_cast<f32x4 *>(&smp->ref[t][c0]) = f32x4{carry[0], carry[1], carry[2], carry[3]};
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bf16x4 kp;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                kp[i] = (bf16)((float)kv[t][i] * __expf(carry[i] - G[t][i]));
            *reinterpret_cast<bf16x4 *>(&smp->p.KP[16 * t + m][c0]) = kp;
        }
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 1: value block w.  O^T = S^T Q^^T + O0^T and U^T = U~^T - S^T W^T
    // (row layout), then the gate: dZ = dY O s (1 - s), dO = dY s, s = sigmoid(Z)
    {
        f32x4 o[4], u[4];
#pragma unroll
        for (int tp = 0; tp < 2; ++tp) {
            const bf16x8 x = gload<bf16x8>(rf, kOffO0 + w * 2048 +
                                                               tp * 1024 + lane * 16);
            o[2 * tp] = f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
            o[2 * tp + 1] = f32x4{(float)x[4], (float)x[5], (float)x[6], (float)x[7]};
        }
        bf16x4 zb[4], yb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            u[t] = f4(gload<bf16x4>(rf, kOffXU + (t * 4 + (w >> 1)) * kFragBytes +
                                                       lane * 16 + (w & 1) * 8));
            zb[t] = gload<bf16x4>(gz, roff(t));
            yb[t] = gload<bf16x4>(gy, roff(t));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                o[t] = mfma16(sf[ks], smp->a.f.QH[t * 4 + ks][lane], o[t]);
                ws = mfma16(sf[ks], smp->a.f.W[t * 4 + ks][lane], ws);
            }
            u[t] -= ws;
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const bool ok = 16 * t + m < len;
            bf16x4 dz4, do4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-(float)zb[t][i]));
                const float dy = ok ? (float)yb[t][i] : 0.f;
                dz4[i] = (bf16)(dy * o[t][i] * sg * (1.f - sg));
                do4[i] = (bf16)(dy * sg);
            }
            if (ok)
                gstore(oz, roff(t), dz4);
            *reinterpret_cast<bf16x4 *>(&smp->d.d.DO[16 * t + m][c0]) = do4;
            *reinterpret_cast<bf16x4 *>(&smp->d.d.U[16 * t + m][c0]) = bf4(u[t]);
        }
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // S and dS' as [dk][dv] tiles for the sums over dv (the fragments' space is free)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            smp->a.s.Sb[perm_row(ks, b, e)][16 * w + m] = sf[ks][e];
            smp->a.s.dSb[perm_row(ks, b, e)][16 * w + m] = df[ks][e];
        }
    // dU^T = dS'^T K'^T + dO^T P (row layout, value block w); dO enters in
    // accumulator order as the operand of the product over tokens
    {
        bf16x4 doa[4];
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                doa[s][i] = smp->d.d.DO[16 * s + 4 * b + i][16 * w + m];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                a = mfma16(df[ks], perm8(&smp->p.KP[16 * t + m][0], ks, b), a);
#pragma unroll
            for (int s = t; s < 4; ++s)
                a = mfma16k16(doa[s],
                              *reinterpret_cast<const bf16x4 *>(&smp->t.PT[16 * t + m][16 * s + 4 * b]),
                              a);
            *reinterpret_cast<bf16x4 *>(&smp->d.d.DU[16 * t + m][c0]) = bf4(a);
        }
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 2: key block w, sums over the value channels:
    // dQs^T = S dO^T, dK'^T = dS' U^T (row layout), dW = -dU S^T (accumulator order)
    f32x4 aq[4], ak[4], aG[4];              // dq, dk and dG of the lane's elements
    float kpk[4] = {0.f, 0.f, 0.f, 0.f};    // sum over the lane's tokens of K' dK'
    bf16x4 dwa[4];
    const f32x4 Ge = *reinterpret_cast<const f32x4 *>(&smp->ref[3][c0]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        f32x4 a1 = {0.f, 0.f, 0.f, 0.f}, a2 = a1, a3 = a1;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kc = 32 * ks + 8 * b;
            const bf16x8 srow = lds8(&smp->a.s.Sb[16 * w + m][kc]);
            a1 = mfma16(srow, lds8(&smp->d.d.DO[16 * t + m][kc]), a1);
            a2 = mfma16(lds8(&smp->a.s.dSb[16 * w + m][kc]), lds8(&smp->d.d.U[16 * t + m][kc]), a2);
            a3 = mfma16(lds8(&smp->d.d.DU[16 * t + m][kc]), srow, a3);
        }
        dwa[t] = bf4(-a3);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float eG = __expf(G[t][i]), eP = __expf(Ge[i] - G[t][i]);
            const float qs = scale * (float)qv[t][i] * eG, kp = (float)kv[t][i] * eP;
            aq[t][i] = scale * eG * a1[i];
            ak[t][i] = eP * a2[i];
            aG[t][i] = qs * a1[i] - kp * a2[i];
            kpk[i] += kp * a2[i];
        }
    }
    {
        // e^Ge rowsum(dS' S) of key channel 16 w + m, 32 value channels per lane group
        float pr = 0.f;
#pragma unroll
        for (int pp = 0; pp < 4; ++pp) {
            const bf16x8 sv = lds8(&smp->a.s.Sb[16 * w + m][32 * b + 8 * pp]);
            const bf16x8 dv8 = lds8(&smp->a.s.dSb[16 * w + m][32 * b + 8 * pp]);
#pragma unroll
            for (int e = 0; e < 8; ++e)
                pr += (float)sv[e] * (float)dv8[e];
        }
        pr += __shfl_xor(pr, 16);
        pr += __shfl_xor(pr, 32);
        if (b == 0)
            smp->dgeD[16 * w + m] = gload<float>(rf, kOffDEC + 4 * (16 * w + m)) * pr;
    }
    // dP = lower_incl(dO U^T), 16 x 16 blocks; the blocks stay in registers
    // for their transposed copy (phase 3: its space is still in use)
    f32x4 dpb[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        dpb[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (nb == 1 && w >= 2)
            break;
        int I, J;
        lower_block(w, nb, I, J);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kc = 32 * ks + 8 * b;
            a = mfma16(lds8(&smp->d.d.DO[16 * I + m][kc]), lds8(&smp->d.d.U[16 * J + m][kc]), a);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * I + 4 * b + i, col = 16 * J + m;
            a[i] = (J < I || col <= row) ? a[i] : 0.f;
            smp->p.dP[row][col] = a[i];
        }
        dpb[nb] = a;
    }
    {
        // T^T into P^T's space (P^T was last read before the previous barrier)
        const int r = tid >> 3, c8 = 8 * (tid & 7);
        *reinterpret_cast<bf16x8 *>(&smp->t.TT[r][c8]) =
            gload<bf16x8>(rf, kOffXT + (size_t)(r * kChunk + c8) * 2);
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 3: dQr (dq complete); dX^T = dW^T T (key block w) and
    // dY~^T = dU^T T (value block w), row layout; dv = beta dY~, dKs = beta dX
    float pb[4] = {0.f, 0.f, 0.f, 0.f};     // dbeta terms of the lane's tokens, its 4 channels
    // dP^T: block element (row 16 I + 4 b + i, column 16 J + m) of the lane is
    // element i of the transposed row 16 J + m (one 16-byte store)
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
        if (nb == 1 && w >= 2)
            break;
        int I, J;
        lower_block(w, nb, I, J);
        *reinterpret_cast<f32x4 *>(&smp->a.x.dPT[16 * J + m][16 * I + 4 * b]) = dpb[nb];
    }
    {
        bf16x4 dua[4], vv[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                dua[s][i] = smp->d.d.DU[16 * s + 4 * b + i][16 * w + m];
            vv[s] = gload<bf16x4>(gv_, roff(s));
        }
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            f32x4 dx = {0.f, 0.f, 0.f, 0.f}, dy = dx;
#pragma unroll
            for (int s = t; s < 4; ++s) {
                const bf16x4 tt =
                    *reinterpret_cast<const bf16x4 *>(&smp->t.TT[16 * t + m][16 * s + 4 * b]);
                dx = mfma16k16(dwa[s], tt, dx);
                dy = mfma16k16(dua[s], tt, dy);
            }
            const bool ok = 16 * t + m < len;
            const float br = smp->beta[16 * t + m];
            bf16x4 dv4;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float eG = __expf(G[t][i]);
                const float ks = (float)kv[t][i] * eG;
                dv4[i] = (bf16)(br * dy[i]);
                ak[t][i] += eG * br * dx[i];
                aG[t][i] += ks * br * dx[i];
                pb[t] += dx[i] * ks + dy[i] * (ok ? (float)vv[t][i] : 0.f);
            }
            if (ok)
                gstore(ov, roff(t), dv4);
            *reinterpret_cast<bf16x4 *>(&smp->a.x.DX[16 * t + m][c0]) = bf4(dx);
            *reinterpret_cast<bf16x4 *>(&smp->a.x.DY[16 * t + m][c0]) = bf4(dy);
        }
    }
    // The products over tokens with the blocks of dP (here) and dA (phase 5)
    // run on fp32 factors: every pair of rows (r, s) of A and P adds a term to
    // dG_r and its negative to dG_s, which cancel in the suffix sums of dg, so
    // both must come from the same fp32 values.  Block (I, J) takes the column
    // factors K_J e^{B_I - G_J} for the row gradients (at most 1 off the
    // diagonal blocks, e^80 on them).
    {
        // k and G in accumulator order (channel 16 w + m), transposed from the
        // row layout; Ba[t] = G before tile t of that channel
        bf16x4 ka[4];
        f32x4 Ga[4];
        float Ba[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ka[t] = acc_order(kv[t], b, m);
            Ga[t] = acc_order(f32x4{G[t][0], G[t][1], G[t][2], G[t][3]}, b, m);
            Ba[t] = t == 0 ? 0.f : smp->ref[t - 1][16 * w + m];
        }
        // dQr^T = (dP Kc)^T for row tile I, then dq = scale (e^G dQs + e^{G-B} dQr)
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 ap = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const f32x4 pr =
                    *reinterpret_cast<const f32x4 *>(&smp->p.dP[16 * I + m][16 * J + 4 * b]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    ap = mfma4_f32((float)ka[J][kk] * __expf(Ba[I] - Ga[J][kk]), pr[kk], ap);
            }
            const f32x4 Bi = ref4(*smp, I, c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float eGB = __expf(G[I][i] - Bi[i]);
                aq[I][i] += scale * eGB * ap[i];
                aG[I][i] += scale * (float)qv[I][i] * eGB * ap[i];
            }
            if (16 * I + m < len)
                gstore(oq, roff(I), bf4(aq[I]));
        }
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 4: dA = strict_lower(-dX W^T - dY~ U~^T), 16 x 16 blocks ------
    for (int nb = 0; nb < (w < 2 ? 2 : 1); ++nb) {
        int I, J;
        lower_block(w, nb, I, J);
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const size_t off = (J * 4 + ks) * kFragBytes + lane * 16;
            const bf16x8 wfr = gload<bf16x8>(rf, kOffXW + off);
            const bf16x8 ufr = gload<bf16x8>(rf, kOffXU + off);
            a = mfma16(perm8(&smp->a.x.DX[16 * I + m][0], ks, b), wfr, a);
            a = mfma16(perm8(&smp->a.x.DY[16 * I + m][0], ks, b), ufr, a);
        }
        f32x4 bt;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * I + 4 * b + i, col = 16 * J + m;
            const float x = (J < I || col < row) ? -a[i] : 0.f;
            smp->a.x.dA[row][col] = x;
            bt[i] = smp->beta[row] * x;
        }
        *reinterpret_cast<f32x4 *>(&smp->d.dAbT[16 * J + m][16 * I + 4 * b]) = bt;
    }
    __syncthreads();

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 5: the products over tokens with the blocks of dA (and dP for
    // the column gradients), fp32, as in phase 3.  Block (I, J) takes the row
    // factors K_I e^{G_I - B_J}, q_I e^{G_I - B_J} for the column gradients;
    // their operands (diag(beta) dA)^T and dP^T are read as rows of the
    // transposed copies.
    {
        bf16x4 ka[4], qa[4];
        f32x4 Ga[4];
        float Ba[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            ka[t] = acc_order(kv[t], b, m);
            qa[t] = acc_order(qv[t], b, m);
            Ga[t] = acc_order(f32x4{G[t][0], G[t][1], G[t][2], G[t][3]}, b, m);
            Ba[t] = t == 0 ? 0.f : smp->ref[t - 1][16 * w + m];
        }
        // row gradients: Z^T = (dA Kc)^T for row tile I, dKr = diag(beta) Z
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 az = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int J = 0; J <= I; ++J) {
                const f32x4 ar = *reinterpret_cast<const f32x4 *>(&smp->a.x.dA[16 * I + m][16 * J + 4 * b]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    az = mfma4_f32((float)ka[J][kk] * __expf(Ba[I] - Ga[J][kk]), ar[kk], az);
            }
            const float br = smp->beta[16 * I + m];
            const f32x4 Bi = ref4(*smp, I, c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float eGB = __expf(G[I][i] - Bi[i]);
                const float kr = (float)kv[I][i] * eGB;
                ak[I][i] += eGB * br * az[i];
                aG[I][i] += kr * br * az[i];
                pb[I] += kr * az[i];
            }
        }
        // column gradients: dKc^T = ((beta dA)^T Kr + dP^T Qr)^T for column tile J
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = J; I < 4; ++I) {
                const f32x4 ab = *reinterpret_cast<const f32x4 *>(&smp->d.dAbT[16 * J + m][16 * I + 4 * b]);
                const f32x4 pt = *reinterpret_cast<const f32x4 *>(&smp->a.x.dPT[16 * J + m][16 * I + 4 * b]);
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float e = __expf(Ga[I][kk] - Ba[J]);
                    a = mfma4_f32((float)ka[I][kk] * e, ab[kk], a);
                    a = mfma4_f32(scale * (float)qa[I][kk] * e, pt[kk], a);
                }
            }
            const f32x4 Bj = ref4(*smp, J, c0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float eBG = __expf(Bj[i] - G[J][i]);
                ak[J][i] += eBG * a[i];
                aG[J][i] -= (float)kv[J][i] * eBG * a[i];
            }
        }
    }

    smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
    // ---- phase 6: dbeta, dGe, dg = suffix sums of dG + dGe; stores ------------
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float x = pb[t];
        x += __shfl_xor(x, 16);
        x += __shfl_xor(x, 32);
        if (b == 0)
            smp->dbp[w][16 * t + m] = x;
    }
    {
        float carry[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float x = kpk[i];                  // over the 16 tokens m of the lane's row
            x += __shfl_xor(x, 1);
            x += __shfl_xor(x, 2);
            x += __shfl_xor(x, 4);
            x += __shfl_xor(x, 8);
            carry[i] = smp->dgeD[c0 + i] + x;    // dGe of channel c0 + i
        }
        bf16x4 og[4];
#pragma unroll
        for (int t = 3; t >= 0; --t)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = aG[t][i];
                const float incl = row_inclusive_sum(x);
                const float tot = row_bcast<15>(incl);
                og[t][i] = (bf16)(carry[i] + tot - incl + x);
                carry[i] += tot;
            }
#pragma unroll
        for (int t = 0; t < 4; ++t)
            if (16 * t + m < len) {
                gstore(ok_, roff(t), bf4(ak[t]));
                gstore(og_, roff(t), og[t]);
            }
    }
    __syncthreads();
    if (tid < len) {
        float s = 0.f;
#pragma unroll
        for (int x = 0; x < kGWaves; ++x)
            s += smp->dbp[x][tid];
        dbeta[(tok0 + tid) * H + h] = (bf16)s;
    }
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const bf16 *gate, const bf16 *dout, const int32_t *cu, int N,
                                int T, int H, int64_t n_slots, const uint8_t *ws_f,
                                uint8_t *ws_b, hipStream_t stream)
{
    const hipError_t err = once_per_device<1>([]() -> hipError_t {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kda_bwd_prep_bf16_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)sizeof(BwdPrepSmem));
    });
    if (err != hipSuccess)
        return err;
    if (n_slots <= 0 || H <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(kda_bwd_prep_bf16_kernel, dim3((unsigned)(n_slots * H)), dim3(kBpThreads),
                       sizeof(BwdPrepSmem), stream, gate, dout, cu, N, T, H, ws_f, ws_b);
    return hipGetLastError();
}

hipError_t launch_grad_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                            const bf16 *beta, const bf16 *gate, const bf16 *dout, bf16 *dq,
                            bf16 *dk, bf16 *dv, bf16 *dg, bf16 *dbeta, bf16 *dgate,
                            const int32_t *cu, int N, int T, int H, int64_t n_slots, float scale,
                            uint8_t *ws_f, const uint8_t *ws_b, hipStream_t stream)
{
    const hipError_t err = once_per_device<2>([]() -> hipError_t {
        return hipFuncSetAttribute(reinterpret_cast<const void *>(kda_grad_bf16_kernel),
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)sizeof(GradSmem));
    });
    if (err != hipSuccess)
        return err;
    if (n_slots <= 0 || H <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(kda_grad_bf16_kernel, dim3((unsigned)(n_slots * H)), dim3(kGThreads),
                       sizeof(GradSmem), stream, q, k, v, g, beta, gate, dout, dq, dk, dv, dg,
                       dbeta, dgate, cu, N, T, H, scale, ws_f, ws_b);
    return hipGetLastError();
}

}  // namespace kda
