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
//   2. backward prep (here): records with -L^T, Q^^T dO and dec, stored in
//      reverse chunk order, so that
//   3. the unchanged chain kernel, started from dS_final, yields dS_{j+1} for
//      every chunk (record SB) and dS_0;
//   4. gradient kernel (here): one workgroup per (chunk, head) recomputes the
//      chunk subtile by subtile (16 tokens, so every decay factor stays within
//      exp(+-40) around the subtile midpoint and fp32 / bf16 never overflow):
//      a forward sweep gives the states on entry to subtiles 1..3, a backward
//      sweep from dS_{j+1} gives the gradients of the chunk's tokens.
//
// Algebra of one 16-token subtile with entry state S (r, s its rows; G the
// cumulative log-decay from the subtile start including the row; Ge = G of
// row 15; B = G of row 7):
//   Qs = scale Q e^G, Ks = K e^G, Kp = K e^{Ge-G}, Qr = scale Q e^{G-B},
//   Kr = K e^{G-B}, Kc = K e^{B-G};  M = Kr Kc^T, A = strict_lower(diag(beta) M),
//   P = lower_incl(Qr Kc^T), T = (I + A)^-1, W = T diag(beta) Ks,
//   U~ = T diag(beta) V, U = U~ - W S, O = Qs S + P U, S' = diag(e^Ge) S + Kp^T U.
// Backward, given dS' and dO:
//   dU = Kp dS' + P^T dO,  dS = diag(e^Ge) dS' + Qs^T dO - W^T dU,
//   dKp = U dS'^T, dQs = dO S^T, dW = -dU S^T, dP = lower_incl(dO U^T),
//   dT = dW (diag(beta) Ks)^T + dU (diag(beta) V)^T, dA = strict_lower(-T^T dT T^T),
//   dKs = diag(beta) T^T dW, dV = diag(beta) T^T dU, dKr = diag(beta) dA Kc,
//   dKc = dA^T diag(beta) Kr + dP^T Qr, dQr = dP Kc,
//   dbeta = rowsum((T^T dW) Ks + (T^T dU) V + dA M),
//   dQ = scale (e^G dQs + e^{G-B} dQr), dK = e^G dKs + e^{G-B} dKr + e^{B-G} dKc + e^{Ge-G} dKp,
//   dG = dQs Qs + dQr Qr + dKs Ks + dKr Kr - dKc Kc - dKp Kp,
//   dGe = colsum(dKp Kp) + e^Ge rowsum(dS' S),  dg_u = sum_{r >= u} dG_r + dGe.
// B cancels inside M and P, so it carries no gradient.
#include "kda_internal.h"

#include <mutex>
#include <utility>

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
    const uint8_t *rf = ws_f + (slot * H + h) * (int64_t)kRecBytes;
    uint8_t *rb = ws_b + ((si.slot0 + nch - 1 - j) * H + h) * (int64_t)kRecBytes;
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
constexpr int kRL = kDK + 8;     // bf16 row stride of [16][128] and [128][128] tiles
constexpr int kFL = kDK + 4;     // fp32 row stride of [16][128] tiles
constexpr int kTL = kSub + 8;    // bf16 row stride of transposed [128][16] tiles
constexpr int kSL = kSub + 1;    // fp32 row stride of 16 x 16 matrices

typedef float Sq[kSub][kSL];

// Lane kS of the caller's 16-lane row, to every lane of that row (DPP
// row_newbcast: a VALU move, no LDS traffic).
template <int kS>
__device__ __forceinline__ float row_bcast(float x)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + kS, 0xf, 0xf, false));
}

// Step kS of the in-wave forward substitution for T = (I + A)^-1 in column
// form: lane (b, m) owns T[4 b + i2][m] and A[4 b + i2][m]; once row kS of T is
// final it updates every later row.  Row kS of T comes from row group kS / 4
// by a lane shuffle, A[4 b + i2][kS] from lane kS of the lane's own row.
template <int kS>
__device__ __forceinline__ void tsolve_step(f32x4 &t, const f32x4 &a, int b, int m)
{
    const float ts = __shfl(t[kS & 3], m + 16 * (kS >> 2));
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
        const float ars = row_bcast<kS>(a[i2]);
        if (4 * b + i2 > kS)
            t[i2] -= ars * ts;
    }
}

template <int... kS>
__device__ __forceinline__ void tsolve(f32x4 &t, const f32x4 &a, int b, int m,
                                       std::integer_sequence<int, kS...>)
{
    (tsolve_step<kS>(t, a, b, m), ...);
}

// Column of element [x][r] of a transposed [128][16] tile: the four groups of
// four tokens of a row are XOR-permuted by bits 3..4 of the channel x.  A
// group stays contiguous for the 8-byte MFMA operand reads, while the
// transposed 2-byte writes of 32 consecutive-by-4 channels spread over eight
// banks instead of two.
__device__ __forceinline__ int tcol(int x, int r)
{
    return 4 * ((r >> 2) ^ ((x >> 3) & 3)) + (r & 3);
}

struct GradSmem {
    // small and often-read arrays first, so that their addresses fit the
    // 16-bit offsets of LDS instructions
    Sq M, Tm, P, dP, dTu, dA;
    alignas(16) float Bref[kDK];
    alignas(16) float Ge[kDK];
    alignas(16) float dec[kDK];
    alignas(16) float dGeD[kDK];        // e^Ge rowsum(dS' S)
    alignas(16) float beta[kSub];
    alignas(16) float dbp[kGWaves][kSub];   // per-wave partial sums of dbeta
    alignas(16) bf16 dbst[kSub];        // dbeta of the subtile, staged for its store
    alignas(16) float G[kSub][kFL];     // cumulative log-decay within the subtile
    alignas(16) bf16 Kin[kSub][kRL];    // k and q as given (bf16, exact); the pair factors
    alignas(16) bf16 Qin[kSub][kRL];    // of the 16-token contractions are formed from them
    alignas(16) bf16 Ks[kSub][kRL];
    alignas(16) bf16 V[kSub][kRL];
    alignas(16) bf16 U[kSub][kRL];
    alignas(16) bf16 dO[kSub][kRL];
    alignas(16) bf16 dU[kSub][kRL];
    union {
        struct {                         // operands of the state products
            alignas(16) bf16 Qs[kSub][kRL];
            alignas(16) bf16 Kp[kSub][kRL];
            alignas(16) bf16 QsT[kDK][kTL];
            alignas(16) bf16 KpT[kDK][kTL];
            union {
                struct {                 // bf16 operands of M and P
                    alignas(16) bf16 Kr[kSub][kRL];
                    alignas(16) bf16 Kc[kSub][kRL];
                    alignas(16) bf16 Qr[kSub][kRL];
                } mp;
                struct {                 // written once T exists
                    alignas(16) bf16 W[kSub][kRL];
                    alignas(16) bf16 WT[kDK][kTL];
                } w;
            } x;
        } a;
        struct {
            alignas(16) float dW[kSub][kFL];
        } b;
    } u;
    union {
        struct {
            alignas(16) bf16 Sb[kDK][kRL];      // S on entry to the subtile, [dk][dv]
            alignas(16) bf16 dSb[kDK][kRL];     // dS' on exit of the subtile, [dk][dv]
        } s;
        // once the sums over the value channels are done: the subtile's token
        // gradients dq, dk, dv, dg, dz, staged for row-contiguous stores
        alignas(16) bf16 out[5][kSub][kRL];
    } v;
};
static_assert(sizeof(GradSmem) <= 160 * 1024, "gradient kernel LDS fits one CU");

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

__device__ __forceinline__ bf16x4 bf4(const f32x4 &x)
{
    return bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
}

// Zero, hidden from the optimizer (an empty asm statement that only claims to
// modify the value; no instruction is emitted).  Adding it to the LDS base at
// the top of every pass keeps the compiler from hoisting the several dozen
// loop-invariant LDS addresses of a pass out of the pass loops, where they
// would hold registers for the whole kernel and force spills; recomputing
// them costs a few integer adds per pass.
__device__ __forceinline__ uint32_t opaque_zero()
{
    uint32_t z = 0;
    asm volatile("" : "+s"(z));
    return z;
}

// Inputs of one subtile pass, loaded a pass ahead: row er, channels ec..ec+3
// of k, g, v, q and beta of row er (elementwise mapping), and the gate logits
// and dY of rows 4 b + i, channel col (the wave's mapping).
// The 16-bit values are kept as raw bits, one per register, and converted
// where used: packing or converting them right after the load would make the
// compiler wait for every load in flight.
struct GradIn {
    bf16x4 k, g, v, q;
    uint16_t beta;
    uint16_t z[4], dy[4];
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t x)
{
    return __uint_as_float((uint32_t)x << 16);
}

// Layout of the per-wave tiles below: wave w owns key (or value) channels
// 16 w .. 16 w + 15; lane (b, m) = (lane / 16, lane % 16) holds rows 4 b + i
// (i = 0..3) of channel 16 w + m, the accumulator layout of the 16x16 MFMAs.
// A chunk is worked in passes over its 16-token subtiles: forward passes
// 0 .. nsub - 2 (states on entry to subtiles 1 .. nsub - 1), then backward
// passes nsub - 1 .. 0.
__global__ __launch_bounds__(kGThreads) void kda_grad_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, const bf16 *__restrict__ gate,
    const bf16 *__restrict__ dout, bf16 *__restrict__ dq, bf16 *__restrict__ dk,
    bf16 *__restrict__ dv, bf16 *__restrict__ dg, bf16 *__restrict__ dbeta,
    bf16 *__restrict__ dgate, const int32_t *__restrict__ cu, int N, int T, int H, float scale,
    uint8_t *__restrict__ ws_f, const uint8_t *__restrict__ ws_b)
{
    extern __shared__ __align__(16) uint8_t smem_raw[];
    // re-derived from an opaque zero at the top of every pass (see opaque_zero)
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
    const int nsub = (len + kSub - 1) / kSub;
    const int npass = 2 * nsub - 1;
    uint8_t *rf = ws_f + (slot * H + h) * (int64_t)kRecBytes;
    const uint8_t *rb = ws_b + ((si.slot0 + nch - 1 - j) * H + h) * (int64_t)kRecBytes;

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, b = lane >> 4;
    const int col = kVBlock * w + m;                          // the lane's channel
    const int er = tid >> 5, ec = 4 * (tid & 31);            // elementwise: row, 4 channels

    // The state on entry to subtile i as this wave's B fragments (perm order):
    // subtile 0 from the forward record's SB; subtiles 1..nsub-2 are parked in
    // the same record's first 96 KiB (LN, QH, BM, O0, no longer read once the
    // backward records exist), 32 KiB per subtile, each lane reading back only
    // the 16-byte slots it wrote.
    static_assert(kOffDEC >= 3 * 32768, "three parked states fit before DEC");
    auto sfrag_ptr = [&](int i, int ks) -> uint8_t * {
        return i == 0 ? rf + kOffSB + w * 4096 + ks * 1024 + lane * 16
                      : rf + (i - 1) * 32768 + w * 4096 + ks * 1024 + lane * 16;
    };
    auto pass_sub = [&](int p) { return p < nsub - 1 ? p : 2 * nsub - 2 - p; };

    // token inputs of subtile i (q only for a backward pass)
    auto load_tok = [&](GradIn &in, int i, bool bwd) {
        const int r0 = kSub * i;
        const int64_t etok = tok0 + r0 + er;
        const int64_t eoff = (etok * H + h) * (int64_t)kDK + ec;
        in.k = in.g = in.v = in.q = bf16x4{};
        in.beta = 0;
        if (r0 + er < len) {
            in.k = *reinterpret_cast<const bf16x4 *>(k + eoff);
            in.g = *reinterpret_cast<const bf16x4 *>(g + eoff);
            in.v = *reinterpret_cast<const bf16x4 *>(v + eoff);
            if (bwd)
                in.q = *reinterpret_cast<const bf16x4 *>(q + eoff);
            if ((tid & 31) == 0)
                in.beta = reinterpret_cast<const uint16_t *>(beta)[etok * H + h];
        }
    };
    // gate and output gradient of subtile i on the lane's value channel.  A row
    // past the end reads the last row of the chunk (always in range) and is
    // masked where it is used: branch-free loads, so that nothing that depends
    // on a loaded value is scheduled next to its load.
    auto load_gate = [&](GradIn &in, int i) {
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int row = min(kSub * i + 4 * b + i2, len - 1);
            const int64_t off = ((tok0 + row) * H + h) * (int64_t)kDV + col;
            in.z[i2] = reinterpret_cast<const uint16_t *>(gate)[off];
            in.dy[i2] = reinterpret_cast<const uint16_t *>(dout)[off];
        }
    };

    // A pass's token inputs are loaded one pass ahead, as soon as the pass
    // before it has copied its own into LDS; a backward pass's gate, output
    // gradient and state fragments (first needed after the operand set-up) right
    // after that, at the top of the pass itself.  All global stores come after
    // these loads and none at the end of a pass: loads and stores share one
    // in-order counter, so a wait for a load also waits for every store issued
    // before it.
    GradIn cur;
    bf16x8 sf[4];                    // state fragments of the current subtile
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        sf[ks] = *reinterpret_cast<const bf16x8 *>(sfrag_ptr(0, ks));
    load_tok(cur, pass_sub(0), npass == 1);

    // Row-contiguous stores of the token gradients of subtile i staged in LDS
    // (16 bytes per lane: array a, row r, channels 8 c8 ..) and of its dbeta, by
    // the nthr threads rt = 0 .. nthr - 1.  In a backward pass they are issued by
    // waves 2..7 while waves 0 and 1 form M, A, T and P, after the pass's loads,
    // so that no load waits behind them.
    auto store_staged = [&](int i, int rt, int nthr) {
        bf16 *const dst[5] = {dq, dk, dv, dg, dgate};
        const int r0 = kSub * i;
        for (int idx = rt; idx < 5 * kSub * 16; idx += nthr) {
            const int a = idx / (kSub * 16), r = (idx / 16) % kSub, c8 = idx % 16;
            if (r0 + r < len)
                *reinterpret_cast<bf16x8 *>(dst[a] + ((tok0 + r0 + r) * H + h) * (int64_t)kDK +
                                            8 * c8) = lds8(&smp->v.out[a][r][8 * c8]);
        }
        if (rt < kSub && r0 + rt < len)
            dbeta[(tok0 + r0 + rt) * H + h] = smp->dbst[rt];
    };

    // Operands of the subtile of pass p: G, factored K / Q tiles, M, A (P), T,
    // W and U~ (returned).  Issues the next pass's token loads once this pass's
    // tokens are in LDS, then a backward pass's own gate and state loads; in a
    // backward pass after the first, waves 2..7 store the previous pass's staged
    // gradients (subtile i + 1) during the M / A / T / P step.
    auto prep_pass = [&](int p, bool bwd, int i) -> f32x4 {
        if ((tid & 31) == 0)
            smp->beta[er] = bf16_bits_to_f32(cur.beta);
        *reinterpret_cast<f32x4 *>(&smp->G[er][ec]) =
            f32x4{(float)cur.g[0], (float)cur.g[1], (float)cur.g[2], (float)cur.g[3]};
        *reinterpret_cast<bf16x4 *>(&smp->V[er][ec]) = cur.v;
        *reinterpret_cast<bf16x4 *>(&smp->Kin[er][ec]) = cur.k;
        *reinterpret_cast<bf16x4 *>(&smp->Qin[er][ec]) = cur.q;
        if (p + 1 < npass)
            load_tok(cur, pass_sub(p + 1), p + 1 >= nsub - 1);
        if (bwd) {
            load_gate(cur, i);
            if (p > nsub - 1) {      // the first backward pass has S_{nsub-1} in registers
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    sf[ks] = *reinterpret_cast<const bf16x8 *>(sfrag_ptr(i, ks));
            }
        }
        __syncthreads();
        if (tid < kDK) {
            float acc = 0.f;
#pragma unroll
            for (int r = 0; r < kSub; ++r) {
                acc += smp->G[r][tid];
                smp->G[r][tid] = acc;
                if (r == kSub / 2 - 1)
                    smp->Bref[tid] = acc;
            }
            smp->Ge[tid] = acc;
            smp->dec[tid] = __expf(acc);
        }
        __syncthreads();
        {
            bf16x4 ks, kp, qs, kr, kc, qr;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int x = ec + e;
                const float G = smp->G[er][x], d = G - smp->Bref[x], Ge = smp->Ge[x];
                const float eG = __expf(G), eP = __expf(Ge - G), eGB = __expf(d), eBG = __expf(-d);
                const float kv = (float)smp->Kin[er][x], qv = scale * (float)smp->Qin[er][x];
                ks[e] = (bf16)(kv * eG);
                kp[e] = (bf16)(kv * eP);
                qs[e] = (bf16)(qv * eG);
                kr[e] = (bf16)(kv * eGB);
                kc[e] = (bf16)(kv * eBG);
                qr[e] = (bf16)(qv * eGB);
                smp->u.a.KpT[x][tcol(x, er)] = kp[e];
                if (bwd)
                    smp->u.a.QsT[x][tcol(x, er)] = qs[e];
            }
            *reinterpret_cast<bf16x4 *>(&smp->Ks[er][ec]) = ks;
            *reinterpret_cast<bf16x4 *>(&smp->u.a.Kp[er][ec]) = kp;
            *reinterpret_cast<bf16x4 *>(&smp->u.a.x.mp.Kr[er][ec]) = kr;
            *reinterpret_cast<bf16x4 *>(&smp->u.a.x.mp.Kc[er][ec]) = kc;
            if (bwd) {
                *reinterpret_cast<bf16x4 *>(&smp->u.a.Qs[er][ec]) = qs;
                *reinterpret_cast<bf16x4 *>(&smp->u.a.x.mp.Qr[er][ec]) = qr;
            }
        }
        __syncthreads();
        // M = Kr Kc^T, A and T = (I + A)^-1 (wave 0); P = lower_incl(Qr Kc^T) (wave 1)
        if (w == 0 || (bwd && w == 1)) {
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const bf16 *xr = w == 0 ? &smp->u.a.x.mp.Kr[m][0] : &smp->u.a.x.mp.Qr[m][0];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mfma16(lds8(xr + 32 * ks + 8 * b), lds8(&smp->u.a.x.mp.Kc[m][32 * ks + 8 * b]),
                             acc);
            if (w == 0) {
                // lane (b, m) holds A[4 b + i2][m]
                f32x4 a;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    const int r = 4 * b + i2;
                    a[i2] = m < r ? smp->beta[r] * acc[i2] : 0.f;
                    smp->M[r][m] = acc[i2];
                }
                // T = (I + A)^-1 by forward substitution inside the wave
                f32x4 t;
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2)
                    t[i2] = (4 * b + i2 == m) ? 1.f : 0.f;
                tsolve(t, a, b, m, std::make_integer_sequence<int, kSub - 1>{});
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2)
                    smp->Tm[4 * b + i2][m] = t[i2];
            } else {
#pragma unroll
                for (int i2 = 0; i2 < 4; ++i2) {
                    const int r = 4 * b + i2;
                    smp->P[r][m] = m <= r ? acc[i2] : 0.f;
                }
            }
        } else if (bwd && p > nsub - 1) {
            // waves 2..7; the staging area is next written in this pass's U / O step
            store_staged(i + 1, tid - 2 * 64, kGThreads - 2 * 64);
        }
        __syncthreads();
        // W = T diag(beta) Ks and U~ = T diag(beta) V on the wave's channels (fp32 MFMA)
        f32x4 ut;
        {
            f32x4 wt = {0.f, 0.f, 0.f, 0.f}, u = wt;
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const int s = 4 * kk + b;
                const float t = smp->Tm[m][s], bs = smp->beta[s];
                wt = mfma4_f32(t, bs * (float)smp->Ks[s][col], wt);
                u = mfma4_f32(t, bs * (float)smp->V[s][col], u);
            }
            ut = u;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                smp->u.a.x.w.W[4 * b + i2][col] = (bf16)wt[i2];
                smp->u.a.x.w.WT[col][tcol(col, 4 * b + i2)] = (bf16)wt[i2];
            }
        }
        __syncthreads();
        return ut;
    };

    // ---------------- forward passes: states on entry to subtiles 1 .. nsub - 1
    if (nsub > 1) {
        f32x4 S[8];                  // the fp32 state of the wave's value channels
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                S[2 * ks][i] = (float)sf[ks][i];
                S[2 * ks + 1][i] = (float)sf[ks][4 + i];
            }
#pragma unroll 1
        for (int p = 0; p < nsub - 1; ++p) {
            const int i = p;
            smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
            const f32x4 ut = prep_pass(p, false, i);
            // S' = diag(e^Ge) S + Kp^T U, U = U~ - W S
            f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                ws = mfma16(perm8(&smp->u.a.x.w.W[m][0], ks, b), sf[ks], ws);
            const bf16x4 ub = bf4(ut - ws);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 dc = *reinterpret_cast<const f32x4 *>(&smp->dec[16 * t + 4 * b]);
                S[t] = S[t] * dc;
                S[t] = mfma16k16(*reinterpret_cast<const bf16x4 *>(
                                     &smp->u.a.KpT[16 * t + m][tcol(16 * t + m, 4 * b)]),
                                 ub, S[t]);
            }
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                sf[ks] = acc_to_frag(S[2 * ks], S[2 * ks + 1]);
            __syncthreads();
            if (i + 1 < nsub - 1) {       // S_{nsub-1} stays in registers for the first backward pass
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    *reinterpret_cast<bf16x8 *>(sfrag_ptr(i + 1, ks)) = sf[ks];
            }
        }
    }

    // ---------------- backward passes over the subtiles, last to first
    f32x4 dS[8];                     // dS' of the wave's value channels, from the backward record
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
        const bf16x8 d = *reinterpret_cast<const bf16x8 *>(rb + kOffSB + w * 4096 + ks * 1024 +
                                                           lane * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            dS[2 * ks][i] = (float)d[i];
            dS[2 * ks + 1][i] = (float)d[4 + i];
        }
    }
#pragma unroll 1
    for (int p = nsub - 1; p < npass; ++p) {
        const int i = pass_sub(p);
        const int r0 = kSub * i;
        smp = reinterpret_cast<GradSmem *>(smem_raw + opaque_zero());
        const f32x4 ut = prep_pass(p, true, i);
        // U and O on the wave's value channels
        f32x4 ws = {0.f, 0.f, 0.f, 0.f}, o = ws;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            ws = mfma16(perm8(&smp->u.a.x.w.W[m][0], ks, b), sf[ks], ws);
            o = mfma16(perm8(&smp->u.a.Qs[m][0], ks, b), sf[ks], o);
        }
        const bf16x4 ub = bf4(ut - ws);
        {
            bf16x4 pa;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pa[e] = (bf16)smp->P[m][4 * b + e];
            o = mfma16k16(pa, ub, o);
        }
        // gate: dZ (kept until the outputs are staged), and dO = dY sigmoid(Z)
        f32x4 dOv;
        bf16x4 dz4;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const float sg = __builtin_amdgcn_rcpf(1.f + __expf(-bf16_bits_to_f32(cur.z[i2])));
            const float dyv = r0 + 4 * b + i2 < len ? bf16_bits_to_f32(cur.dy[i2]) : 0.f;
            dz4[i2] = (bf16)(dyv * o[i2] * sg * (1.f - sg));
            dOv[i2] = dyv * sg;
        }
        const bf16x4 dob = bf4(dOv);
        // dU = Kp dS' + P^T dO
        f32x4 du = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            du = mfma16(perm8(&smp->u.a.Kp[m][0], ks, b), acc_to_frag(dS[2 * ks], dS[2 * ks + 1]),
                        du);
        {
            bf16x4 pt;
#pragma unroll
            for (int e = 0; e < 4; ++e)
                pt[e] = (bf16)smp->P[4 * b + e][m];
            du = mfma16k16(pt, dob, du);
        }
        const bf16x4 dub = bf4(du);
        // U, dO, dU, S and dS' of the wave's value channels into LDS
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int r = 4 * b + i2;
            smp->U[r][col] = ub[i2];
            smp->dO[r][col] = dob[i2];
            smp->dU[r][col] = dub[i2];
        }
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                smp->v.s.Sb[perm_row(ks, b, e)][col] = sf[ks][e];
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                smp->v.s.dSb[16 * t + 4 * b + i2][col] = (bf16)dS[t][i2];
        // dS on entry to the subtile: diag(e^Ge) dS' + Qs^T dO - W^T dU
        __builtin_amdgcn_sched_barrier(0);
        {
            const bf16x4 ndub = bf16x4{(bf16)(-du[0]), (bf16)(-du[1]), (bf16)(-du[2]),
                                       (bf16)(-du[3])};
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                const f32x4 dc = *reinterpret_cast<const f32x4 *>(&smp->dec[16 * t + 4 * b]);
                f32x4 x = dS[t] * dc;
                x = mfma16k16(*reinterpret_cast<const bf16x4 *>(
                                  &smp->u.a.QsT[16 * t + m][tcol(16 * t + m, 4 * b)]),
                              dob, x);
                dS[t] = mfma16k16(
                    *reinterpret_cast<const bf16x4 *>(
                        &smp->u.a.x.w.WT[16 * t + m][tcol(16 * t + m, 4 * b)]), ndub, x);
            }
        }
        __syncthreads();

        // sums over the value channels on the wave's key channels col:
        // dKp = U dS'^T, dQs = dO S^T, dW = -dU S^T
        f32x4 dkp = {0.f, 0.f, 0.f, 0.f}, dqs = dkp, dw = dkp;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int kc = 32 * ks + 8 * b;
            const bf16x8 srow = lds8(&smp->v.s.Sb[col][kc]);
            dkp = mfma16(lds8(&smp->U[m][kc]), lds8(&smp->v.s.dSb[col][kc]), dkp);
            dqs = mfma16(lds8(&smp->dO[m][kc]), srow, dqs);
            dw = mfma16(lds8(&smp->dU[m][kc]), srow, dw);
        }
        dw = -dw;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2)
            smp->u.b.dW[4 * b + i2][col] = dw[i2];
        {
            // e^Ge rowsum(dS' S) of key channel col, 32 value channels per lane group
            float pr = 0.f;
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
                const bf16x8 sv = lds8(&smp->v.s.Sb[col][32 * b + 8 * pp]);
                const bf16x8 dv8 = lds8(&smp->v.s.dSb[col][32 * b + 8 * pp]);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    pr += (float)sv[e] * (float)dv8[e];
            }
            pr += __shfl_xor(pr, 16);
            pr += __shfl_xor(pr, 32);
            if (b == 0)
                smp->dGeD[col] = smp->dec[col] * pr;
        }
        if (w == 0 || w == 1) {
            // wave 0: dP = lower_incl(dO U^T); wave 1: dU (diag(beta) V)^T
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
            const bf16 *ar = w == 0 ? &smp->dO[m][0] : &smp->dU[m][0];
            const bf16 *br = w == 0 ? &smp->U[m][0] : &smp->V[m][0];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                acc = mfma16(lds8(ar + 32 * ks + 8 * b), lds8(br + 32 * ks + 8 * b), acc);
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                const int r = 4 * b + i2;
                if (w == 0)
                    smp->dP[r][m] = m <= r ? acc[i2] : 0.f;
                else
                    smp->dTu[r][m] = smp->beta[m] * acc[i2];
            }
        }
        __syncthreads();
        // dT = dW (diag(beta) Ks)^T + dU (diag(beta) V)^T, then
        // dA = strict_lower(-T^T (dT T^T)), all in wave 0 and in registers: an
        // accumulator tile (lane (b, n) holds D[4 b + i][n]) is used directly as
        // the next 16x16x4 product's operand, with the contraction index of step
        // kk taken as k = 4 b + kk on both sides
        if (w == 0) {
            // dT^T: lane (b, m) holds dT[m][4 b + i]
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int kc = 32 * ks + 8 * b;
                const f32x4 lo = *reinterpret_cast<const f32x4 *>(&smp->u.b.dW[m][kc]);
                const f32x4 hi = *reinterpret_cast<const f32x4 *>(&smp->u.b.dW[m][kc + 4]);
                acc = mfma16(lds8(&smp->Ks[m][kc]), acc_to_frag(lo, hi), acc);
            }
            f32x4 dtt;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                dtt[i2] = smp->beta[4 * b + i2] * acc[i2] + smp->dTu[m][4 * b + i2];
            // Y = dT T^T: A[m][k] = dT[m][k] is dtt[kk], B[k][n] = T[n][k]
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                y = mfma4_f32(dtt[kk], smp->Tm[m][4 * b + kk], y);
            // T^T Y: A[m][k] = T[k][m], B[k][n] = Y[k][n] is y[kk]
            f32x4 x2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                x2 = mfma4_f32(smp->Tm[4 * b + kk][m], y[kk], x2);
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                const int r = 4 * b + i2;
                smp->dA[r][m] = m < r ? -x2[i2] : 0.f;
            }
        }
        __syncthreads();

        // the contractions over the subtile's 16 tokens, on the wave's channels:
        // T^T dW, T^T dU, dP^T Qr + dA^T diag(beta) Kr, dA Kc, dP Kc.  Kr, Kc and
        // Qr enter in fp32: every pair (r, s) of A and P adds a term to dG_r and
        // its negative to dG_s, and the two cancel in the reverse cumulative sum
        // that gives dg, so both must be formed from the same fp32 factors.
        f32x4 tdw = {0.f, 0.f, 0.f, 0.f}, tdu = tdw, dkc = tdw, dkr = tdw, dqr = tdw;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const int s = 4 * kk + b;
            const float t_ms = smp->Tm[s][m];
            const float d = smp->G[s][col] - smp->Bref[col];
            const float egb = __expf(d), ebg = __expf(-d);
            const float ks_ = (float)smp->Kin[s][col];
            const float kc_s = ks_ * ebg, kr_s = ks_ * egb;
            const float qr_s = scale * (float)smp->Qin[s][col] * egb;
            tdw = mfma4_f32(t_ms, smp->u.b.dW[s][col], tdw);
            tdu = mfma4_f32(t_ms, (float)smp->dU[s][col], tdu);
            dkc = mfma4_f32(smp->dP[s][m], qr_s, dkc);
            dkc = mfma4_f32(smp->dA[s][m] * smp->beta[s], kr_s, dkc);
            dkr = mfma4_f32(smp->dA[m][s], kc_s, dkr);
            dqr = mfma4_f32(smp->dP[m][s], kc_s, dqr);
        }
        // per element: row r = 4 b + i2, channel col (all reads first, stores last)
        float dGv[4], pb[4], kpk = 0.f;
        bf16x4 oq, ok, ov;
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int r = 4 * b + i2;
            const float kv = (float)smp->Kin[r][col];
            const float qv = scale * (float)smp->Qin[r][col];
            const float G = smp->G[r][col], d = G - smp->Bref[col], Ge = smp->Ge[col];
            const float eG = __expf(G), eGB = __expf(d), eBG = __expf(-d), eP = __expf(Ge - G);
            const float br = smp->beta[r];
            const float dks = br * tdw[i2], dkr_ = br * dkr[i2];
            oq[i2] = (bf16)(scale * (eG * dqs[i2] + eGB * dqr[i2]));
            ok[i2] = (bf16)(eG * dks + eGB * dkr_ + eBG * dkc[i2] + eP * dkp[i2]);
            ov[i2] = (bf16)(br * tdu[i2]);
            dGv[i2] = dqs[i2] * qv * eG + dqr[i2] * qv * eGB + dks * kv * eG + dkr_ * kv * eGB -
                      dkc[i2] * kv * eBG - dkp[i2] * kv * eP;
            kpk += dkp[i2] * kv * eP;
            // dbeta terms of this element; wave 0 adds the dA M term of row r (its lane
            // m is the column of A)
            pb[i2] = tdw[i2] * kv * eG + tdu[i2] * (float)smp->V[r][col];
            if (w == 0)
                pb[i2] += smp->dA[r][m] * smp->M[r][m];
        }
        // sums of pb over the wave's 16 channels for the lane group's four rows, as
        // a butterfly that also spreads the rows: afterwards lanes with m % 4 == 0
        // hold the sum of row 4 b + 2 ((m >> 3) & 1) + ((m >> 2) & 1)
        {
            const bool hi = (m & 8) != 0, mid = (m & 4) != 0;
            const float a0 = (hi ? pb[2] : pb[0]) + __shfl_xor(hi ? pb[0] : pb[2], 8);
            const float a1 = (hi ? pb[3] : pb[1]) + __shfl_xor(hi ? pb[1] : pb[3], 8);
            float c = (mid ? a1 : a0) + __shfl_xor(mid ? a0 : a1, 4);
            c += __shfl_xor(c, 2);
            c += __shfl_xor(c, 1);
            if ((m & 3) == 0)
                smp->dbp[w][4 * b + 2 * (hi ? 1 : 0) + (mid ? 1 : 0)] = c;
        }
#pragma unroll
        for (int i2 = 0; i2 < 4; ++i2) {
            const int r = 4 * b + i2;
            smp->v.out[0][r][col] = oq[i2];
            smp->v.out[1][r][col] = ok[i2];
            smp->v.out[2][r][col] = ov[i2];
            smp->v.out[4][r][col] = dz4[i2];
        }
        // dg_u = sum_{r >= u} dG_r + dGe with dGe = dGeD + colsum(dKp Kp): the rows of
        // channel col are spread over the four lane groups b
        {
            kpk += __shfl_xor(kpk, 16);
            kpk += __shfl_xor(kpk, 32);
            float suf[4];
            suf[3] = dGv[3];
#pragma unroll
            for (int i2 = 2; i2 >= 0; --i2)
                suf[i2] = suf[i2 + 1] + dGv[i2];
            const float t1 = __shfl(suf[0], m + 16 * ((b + 1) & 3));
            const float t2 = __shfl(suf[0], m + 16 * ((b + 2) & 3));
            const float t3 = __shfl(suf[0], m + 16 * ((b + 3) & 3));
            const float later = (b < 3 ? t1 : 0.f) + (b < 2 ? t2 : 0.f) + (b < 1 ? t3 : 0.f);
            const float dge = smp->dGeD[col] + kpk + later;
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2)
                smp->v.out[3][4 * b + i2][col] = (bf16)(dge + suf[i2]);
        }
        __syncthreads();
        if (tid < kSub) {
            float acc = 0.f;
#pragma unroll
            for (int x = 0; x < kGWaves; ++x)
                acc += smp->dbp[x][tid];
            smp->dbst[tid] = (bf16)acc;
        }
    }
    store_staged(0, tid, kGThreads);
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const bf16 *gate, const bf16 *dout, const int32_t *cu, int N,
                                int T, int H, int64_t n_slots, const uint8_t *ws_f,
                                uint8_t *ws_b, hipStream_t stream)
{
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_bwd_prep_bf16_kernel),
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
    static std::once_flag once;
    static hipError_t err = hipSuccess;
    std::call_once(once, [] {
        err = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_grad_bf16_kernel),
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
