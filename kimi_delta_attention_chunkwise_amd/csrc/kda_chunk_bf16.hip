// kda_chunk_bf16.hip -- chunkwise-parallel KDA forward for bf16 inputs,
// dk = dv = 128, 64-token chunks in four 16-token subtiles, fp32 state.
//
// Sources: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
// section 1 rows Q04/Q05 (channel-wise decay, delta-rule write), Q06
// (log-decay floor g_min = -5 bounds the reciprocal of the cumulative decay,
// so the diagonal tiles can also be bf16 dense products), Q07 (state passed
// recurrently between chunks, matrices within a chunk), Q08 (output gate);
// "Kimi K3 report reveals training and systems stack", confirmed list
// (FlashKDA; chunks further cut into 16-token tiles for stability).
//
// Chunk algebra (derived from the recurrence; r, s are rows of one chunk,
// G_r = sum_{u <= r} g_u per key channel from the chunk start, S the state on
// entry to the chunk):
//   A   = strict_lower(diag(beta) [k_r e^{G_r - G_s} k_s])
//   P   = scale * lower_incl([q_r e^{G_r - G_s} k_s])
//   T   = (I + A)^-1
//   W   = T diag(beta) (K e^G),   U~ = T diag(beta) V,   K' = K e^{G_end - G}
//   U   = U~ - W S
//   O   = scale (Q e^G) S + P U  = Q^ S + O0,   Q^ = scale Q e^G - P W,  O0 = P U~
//   S' = diag(e^{G_end}) S + K'^T U = diag(dec) S + Bm - L S,
//        L = K'^T W,  Bm = K'^T U~,  dec = e^{G_end}
//   y   = sigmoid(z) O
// Only A and P need e^{-G}.  Block (i, j) of A and P (16 x 16, j <= i) uses
// the reference B_i = G at the end of subtile i - 1: rows carry
// e^{G_r - B_i} in [e^-80, 1] and columns carry e^{B_i - G_s}, which is at most
// e^80 on the diagonal block and at most 1 below it, so every bf16 operand
// stays inside the bf16/fp32 exponent range because g >= -5 and a subtile is
// 16 tokens (5 * 16 = 80 < ln(FLT_MAX) = 88.7).  Below the diagonal the
// column factor is formed as e^{B_j - G_s} e^{B_i - B_j}.
//
// Three kernels, in stream order:
//   prep   (persistent, 512 threads per CU, over the (chunk slot, head)
//          tasks; all chunks in parallel): G, A and P (bf16 MFMA), T (fp32
//          substitution and fp32 MFMA), W and U~ (MFMA), then L, Bm, Q^ and O0
//          (MFMA) written to the chunk's workspace record as the later kernels'
//          operand fragments.
//   chain  (640 threads per (sequence, head, 16-wide value block)): walks the
//          chunks in order and carries only the state.  Compute wave w (of 8)
//          keeps rows 16 w .. 16 w + 15 of the fp32 state slice in its
//          accumulators and computes those rows of S' = dec S + Bm - L S; the
//          compute waves exchange the new state as bf16 MFMA fragments through
//          LDS, one barrier per chunk, with their rows of L for the next chunks
//          prefetched into registers.  A side wave loads Bm and the decay of
//          the chunks ahead into LDS, and a store wave copies each chunk's entry
//          state fragments from LDS to the record, so no wave has both loads and
//          stores in flight.
//   output (256 threads per (chunk slot, head)): O = Q^ S + O0 from the
//          record, gated by sigmoid(z), rounded to bf16; all chunks in parallel.
#include "kda_internal.h"

#include <mutex>
#include <numeric>

namespace kda {

namespace {

constexpr int kPrepThreads = 512;
constexpr int kRowLd = 136;   // bf16 row stride of row-major 64 x 128 tiles
constexpr int kColLd = 72;    // bf16 row stride of channel-major 128 x 64 tiles
constexpr int kALd = 68;      // fp32 row stride of A and T: 16-byte rows, and the column
                              // reads of phases 2 and 4 spread over all LDS banks

struct PrepSmem {
    // -- live in phases 1-2 only; T reuses this space afterwards
    bf16 KR[kChunk][kRowLd];      // k e^{G - B_i(r)}      (row operand of A)
    bf16 KCD[kChunk][kRowLd];     // k e^{B_i(r) - G}      (column operand, diagonal ref.)
    float F[6][kDK];              // e^{B_i - B_j}, i > j  (pairs 10 20 21 30 31 32)
    // -- live until the end
    bf16 QR[kChunk][kRowLd];      // q e^{G - B_i(r)}      (row operand of P; Q e^G later)
    bf16 XB[kDK][kColLd];         // beta k e^G, channel-major
    bf16 VB[kDV][kColLd];         // beta v, channel-major
    bf16 KPT[kDK][kColLd];        // K' = k e^{G_end - G}, channel-major
    bf16 PM[kChunk][kColLd];      // scale P, lower incl., zero above
    float AM[kChunk][kALd];       // diag(beta) A, strict lower
    // per-subtile channel constants; rows padded to 132 floats so that the
    // 16-byte reads of four rows by one 16-lane group use different LDS banks
    float eB[4][kDK + 4];         // e^{B_i}
    float eGB[4][kDK + 4];        // e^{G_end - B_i}
    float Gref[4][kDK + 4];       // G at the end of subtiles 0, 1, 2, 3 (B_1, B_2, B_3, G_end)
    float NRM[2][8][kChunk];      // prologue: per-wave partial sums of q^2 and k^2 per row
    float DEC0[kDK];              // pairs: e^{G_end} of chunk 0, kept for chunk 1
};
static_assert(sizeof(PrepSmem) <= 160 * 1024, "prep LDS fits one CU");

// the backward's dO^T tile ([dv][token], kColLd stride) overlays KCD and F
static_assert(offsetof(PrepSmem, F) + sizeof(PrepSmem::F) - offsetof(PrepSmem, KCD) >=
                  sizeof(bf16) * kDV * kColLd,
              "dO^T fits in KCD and F");

struct TSmem {                    // overlays KR after phase 2
    float TM[kChunk][kALd];
};
static_assert(sizeof(TSmem) <= sizeof(bf16) * kChunk * kRowLd, "T overlay fits");

__device__ __forceinline__ int pair_index(int i, int j) { return (i * (i - 1)) / 2 + j; }

// KR, QR and KCD store the 16-byte slot o (channels 8 o .. 8 o + 7) of row r at
// slot o ^ ((r >> 4) & 3).  Phase 1 writes 8 bytes of 16 rows four apart per 16
// lanes; unpermuted, the 68-dword row stride puts them in two LDS banks,
// permuted in eight.  Reads of a whole slot, by rows of one 16-row tile, are
// unaffected.  Column of channel group c4 (channels 4 c4 .. 4 c4 + 3) of row r:
__device__ __forceinline__ int rq(int r, int c4) { return 4 * (c4 ^ ((r >> 3) & 6)); }

// channels 8 o .. 8 o + 7 of row r of such a tile
__device__ __forceinline__ bf16x8 lds8_rq(const bf16 (*t)[kRowLd], int r, int o)
{
    return lds8(&t[r][8 * (o ^ ((r >> 4) & 3))]);
}

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4 &a, float s)
{
    return bf16x4{(bf16)(s * a[0]), (bf16)(s * a[1]), (bf16)(s * a[2]), (bf16)(s * a[3])};
}


}  // namespace

// Inputs of one prep task held in registers: lane (tg, cq) of wave w has
// tokens 4 tg .. 4 tg + 3 of the chunk and key / value channels
// 16 w + 4 cq .. 16 w + 4 cq + 3 (tg = lane % 16, cq = lane / 16).
struct PrepIn {
    bf16x4 q[4], k[4], v[4], g[4];   // [token within the group]
    bf16 beta[4];
};

// One (chunk slot, head) task of the prep kernel.
struct PrepTask {
    bool valid;                      // false: padding slot of the varlen bound
    int h;
    int len;                         // tokens in the chunk, 1 .. 64
    int64_t tok0;                    // first token
    int64_t rec;                     // record index: slot * H + h
    int64_t brec;                    // backward record index: the chunk's slot mirrored
                                     // within its sequence (see the backward), * H + h
};

__device__ __forceinline__ PrepTask prep_task(const int32_t *cu, int N, int T, int H, int64_t t)
{
    // slot-major task order: t = slot * H + h
    PrepTask pt;
    const int64_t slot = t / H;
    pt.h = (int)(t % H);
    pt.rec = t;
    int n;
    int64_t j;
    pt.valid = slot_to_chunk(cu, N, T, slot, n, j);
    pt.len = 0;
    pt.tok0 = 0;
    pt.brec = 0;
    if (pt.valid) {
        const SeqInfo si = seq_info(cu, n, T, kChunk);
        pt.tok0 = si.bos + j * kChunk;
        pt.len = (int)((si.len - j * kChunk) < kChunk ? (si.len - j * kChunk) : kChunk);
        pt.brec = (si.slot0 + (si.len + kChunk - 1) / kChunk - 1 - j) * H + pt.h;
    }
    return pt;
}

// Loads of token t of the lane's group (rows past the end of the chunk
// re-read its last row, so every load stays in the sequence; they are zeroed
// when used).
__device__ __forceinline__ void prep_load_token(PrepIn &in, const bf16 *q, const bf16 *k,
                                                const bf16 *v, const bf16 *g, const bf16 *beta,
                                                const PrepTask &pt, int H, int wave, int tg,
                                                int cq, int t)
{
    const int ch = 16 * wave + 4 * cq;
    const int r = 4 * tg + t < pt.len ? 4 * tg + t : pt.len - 1;
    const int64_t tok = pt.tok0 + r;
    const int64_t off = (tok * H + pt.h) * (int64_t)kDK + ch;
    in.q[t] = *reinterpret_cast<const bf16x4 *>(q + off);
    in.k[t] = *reinterpret_cast<const bf16x4 *>(k + off);
    in.v[t] = *reinterpret_cast<const bf16x4 *>(v + off);
    in.g[t] = *reinterpret_cast<const bf16x4 *>(g + off);
    in.beta[t] = beta[tok * H + pt.h];
}

__device__ __forceinline__ void prep_load(PrepIn &in, const bf16 *q, const bf16 *k, const bf16 *v,
                                          const bf16 *g, const bf16 *beta, const PrepTask &pt,
                                          int H, int wave, int tg, int cq)
{
#pragma unroll
    for (int t = 0; t < 4; ++t)
        prep_load_token(in, q, k, v, g, beta, pt, H, wave, tg, cq, t);
}

// Phases 1 to 5 of one chunk of a prep task.  `in` holds the chunk's inputs on
// entry; while the chunk is in its matrix phases it is refilled with those of
// `next` (when load_next).  kMode selects what is written:
//   0  a chunk record (or a pair record of a sequence's one-chunk last pair):
//      LN, QH, BM, O0 and DEC of the chunk;
//   1  chunk 0 of a pair: its readout QH, O0; -L0 and Bm0 of the wave's 16
//      columns stay in `hold` as B fragments (k = rows, perm order) and its
//      decay in LDS, for chunk 1;
//   2  chunk 1 of a pair: the composed map (LN = -L01, BM = Bm01, DEC = dec01)
//      and its readout from the pair's entry state (QH1, O01).
// kExt (mode 0 in a per-chunk record, never in a pair record): also the
// record's extension XW, XU, XT, XP for the gradient kernel.
// kBwd (with kExt): also the chunk's backward record at brec (LN = -L^T,
// BM = Q^^T dO with dO = dY sigmoid(Z), DEC), what the backward prep kernel
// would form from the forward record.
struct PairHold {
    bf16x8 nl0[4];                   // -L0, column block of the wave, 4 k-steps of rows
    bf16x8 bm0[4];                   // Bm0, the same layout
};

// Operands of the fused backward record (kBwd).
struct BwdOut {
    const bf16 *gate, *dout;         // Z and dY  [.., H, dv]
    uint8_t *rec;                    // the chunk's backward record
};

// A workgroup barrier when data passes between waves, else a wave-level fence
// (LDS operations of one wave take effect in order).  Inside phase 1, G at the
// subtile ends, the per-channel constants and the operands built from them
// pass between lanes of one wave; only the q / k norms of the prologue are
// summed over all waves.
__device__ __forceinline__ void wave_or_group_sync(bool across_waves)
{
    if (across_waves) {
        __syncthreads();
    } else {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

template <bool kPro, int kMode, bool kExt = false, bool kBwd = false>
__device__ __forceinline__ void prep_chunk(PrepSmem &sm, TSmem &ts, PrepIn &in, const bf16 *q,
                                           const bf16 *k, const bf16 *v, const bf16 *g,
                                           const bf16 *beta, const PrepTask &pt,
                                           const PrepTask &next, bool load_next, int H,
                                           float scale, unsigned pro, uint8_t *rec,
                                           PairHold &hold, BwdOut bo = BwdOut{})
{
    static_assert(!kExt || kMode == 0, "the extension belongs to per-chunk records");
    static_assert(!kBwd || kExt, "the backward record comes with a per-chunk record");
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int m = lane & 15, b = lane >> 4;
    const int tg = lane & 15, cq = lane >> 4;     // phase-1 roles: token group, channel quad

    // ---- phase 1: cumulative log-decay and elementwise operands -----------
    // lane (tg, cq): tokens 4 tg .. + 3, channels 16 wave + 4 cq .. + 3
    {
        const int ch0 = 16 * wave + 4 * cq;
        const int ib = tg >> 2;                       // subtile of the lane's tokens
        for (int i = tid; i < kChunk * kColLd / 8; i += kPrepThreads)   // zero P
            reinterpret_cast<bf16x8 *>(&sm.PM[0][0])[i] = bf16x8{};
        // G: inclusive prefix over the lane's 4 tokens, then across the 16
        // token groups of the row (rows past len carry g = 0)
        float G[4][4];                                 // [token][channel]
        float br[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const float bv = (float)in.beta[tt];
            br[tt] = 4 * tg + tt < pt.len ? ((kPro && (pro & kProBeta)) ? sigmoidf_(bv) : bv) : 0.f;
        }
        if (kPro && (pro & kProQK)) {
            // sums of q^2 and k^2 per row: the lane's 4 channels, then the
            // wave's 16 (lanes 16 apart), then the 8 waves through LDS
            float sq[4], sk[4];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                sq[tt] = sk[tt] = 0.f;
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float qv = (float)in.q[tt][c], kv = (float)in.k[tt][c];
                    sq[tt] += qv * qv;
                    sk[tt] += kv * kv;
                }
                sq[tt] += __shfl_xor(sq[tt], 16);
                sq[tt] += __shfl_xor(sq[tt], 32);
                sk[tt] += __shfl_xor(sk[tt], 16);
                sk[tt] += __shfl_xor(sk[tt], 32);
            }
            if (cq == 0) {
                *reinterpret_cast<f32x4 *>(&sm.NRM[0][wave][4 * tg]) =
                    f32x4{sq[0], sq[1], sq[2], sq[3]};
                *reinterpret_cast<f32x4 *>(&sm.NRM[1][wave][4 * tg]) =
                    f32x4{sk[0], sk[1], sk[2], sk[3]};
            }
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            float run = 0.f;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const float x = (float)in.g[tt][c];
                const float gv = (kPro && (pro & kProG)) ? log_decay_from(x) : x;
                run += 4 * tg + tt < pt.len ? gv : 0.f;
                G[tt][c] = run;
            }
            const float excl = row_inclusive_sum(run) - run;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                G[tt][c] += excl;
        }
        // G at the ends of the subtiles: B_1, B_2, B_3 and G_end
        if ((tg & 3) == 3)
            *reinterpret_cast<f32x4 *>(&sm.Gref[ib][ch0]) =
                f32x4{G[3][0], G[3][1], G[3][2], G[3][3]};
        if (wave == 0 && cq == 0) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                sm.AM[4 * tg + tt][kChunk] = br[tt];  // beta per row, for A
        }
        wave_or_group_sync(kPro && (pro & kProQK));
        if (lane < 16) {
            // per-channel constants of channel 16 w + lane
            const int ch = 16 * wave + lane;
            const float b1 = sm.Gref[0][ch], b2 = sm.Gref[1][ch], b3 = sm.Gref[2][ch];
            const float ge = sm.Gref[3][ch];
            sm.eB[0][ch] = 1.f;
            sm.eB[1][ch] = __expf(b1);
            sm.eB[2][ch] = __expf(b2);
            sm.eB[3][ch] = __expf(b3);
            sm.eGB[0][ch] = __expf(ge);
            sm.eGB[1][ch] = __expf(ge - b1);
            sm.eGB[2][ch] = __expf(ge - b2);
            sm.eGB[3][ch] = __expf(ge - b3);
            sm.F[0][ch] = __expf(b1);                    // e^{B_1 - B_0}
            sm.F[1][ch] = __expf(b2);                    // e^{B_2 - B_0}
            sm.F[2][ch] = __expf(b2 - b1);
            sm.F[3][ch] = __expf(b3);
            sm.F[4][ch] = __expf(b3 - b1);
            sm.F[5][ch] = __expf(b3 - b2);
            if constexpr (kMode == 0)
            {
                reinterpret_cast<float *>(rec + kOffDEC)[ch] = __expf(ge);
                if constexpr (kBwd)
                    reinterpret_cast<float *>(bo.rec + kOffDEC)[ch] = __expf(ge);
            }
            else if constexpr (kMode == 1)
                sm.DEC0[ch] = __expf(ge);    // read by chunk 1 of the pair (same lane) and its phase 5
            else
                reinterpret_cast<float *>(rec + kOffDEC)[ch] = sm.DEC0[ch] * __expf(ge);
        }
        wave_or_group_sync(kPro && (pro & kProQK));
        // prologue: 1 / |q| and 1 / |k| of the lane's rows (1 without it)
        f32x4 nq = {1.f, 1.f, 1.f, 1.f}, nk = {1.f, 1.f, 1.f, 1.f};
        if (kPro && (pro & kProQK)) {
            f32x4 aq = {0.f, 0.f, 0.f, 0.f}, ak = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int w2 = 0; w2 < 8; ++w2) {
                aq += *reinterpret_cast<const f32x4 *>(&sm.NRM[0][w2][4 * tg]);
                ak += *reinterpret_cast<const f32x4 *>(&sm.NRM[1][w2][4 * tg]);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                nq[tt] = __builtin_amdgcn_rsqf(aq[tt] + kNormEps);
                nk[tt] = __builtin_amdgcn_rsqf(ak[tt] + kNormEps);
            }
        }
        const f32x4 Bi = ib == 0 ? f32x4{0.f, 0.f, 0.f, 0.f}
                                 : *reinterpret_cast<const f32x4 *>(&sm.Gref[ib - 1][ch0]);
        const f32x4 eb = *reinterpret_cast<const f32x4 *>(&sm.eB[ib][ch0]);
        const f32x4 egb = *reinterpret_cast<const f32x4 *>(&sm.eGB[ib][ch0]);
        bf16x4 xb[4], vb[4], kp[4];                    // [channel][token]
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int r = 4 * tg + tt;
            const bool ok = r < pt.len;
            bf16x4 kr, qr, kc;
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const float fr = __expf(G[tt][c] - Bi[c]);   // e^{G - B_i} in [e^-80, 1]
                const float fc = __builtin_amdgcn_rcpf(fr);  // e^{B_i - G} in [1, e^80]
                const float kv = ok ? (float)in.k[tt][c] * nk[tt] : 0.f;
                const float qv = ok ? (float)in.q[tt][c] * nq[tt] : 0.f;
                const float vv = ok ? (float)in.v[tt][c] : 0.f;
                const float kfr = kv * fr, kfc = kv * fc;
                kr[c] = (bf16)kfr;
                qr[c] = (bf16)(qv * fr);
                kc[c] = (bf16)kfc;
                xb[c][tt] = (bf16)(kfr * eb[c] * br[tt]);          // beta k e^G
                vb[c][tt] = (bf16)(br[tt] * vv);                   // beta v
                kp[c][tt] = (bf16)(kfc * egb[c]);                  // k e^{G_end - G}
            }
            *reinterpret_cast<bf16x4 *>(&sm.KR[r][rq(r, ch0 >> 2)]) = kr;
            *reinterpret_cast<bf16x4 *>(&sm.QR[r][rq(r, ch0 >> 2)]) = qr;
            *reinterpret_cast<bf16x4 *>(&sm.KCD[r][rq(r, ch0 >> 2)]) = kc;
        }
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            *reinterpret_cast<bf16x4 *>(&sm.XB[ch0 + c][4 * tg]) = xb[c];
            *reinterpret_cast<bf16x4 *>(&sm.VB[ch0 + c][4 * tg]) = vb[c];
            *reinterpret_cast<bf16x4 *>(&sm.KPT[ch0 + c][4 * tg]) = kp[c];
        }
    }
    __syncthreads();
    // the registers of this task's inputs are free: fetch the next task's,
    // one token of the lane's group before each of phases 2 to 5, so the
    // loads do not all queue up in front of one phase
    if (load_next)
        prep_load_token(in, q, k, v, g, beta, next, H, wave, tg, cq, 0);

    // ---- phase 2: 16 x 16 blocks of A and P (bf16 MFMA, fp32 accumulate) -------
    // ten blocks on eight waves: the two waves that take two blocks take
    // diagonal ones (no cross-subtile factor to apply), and each of the six
    // off-diagonal blocks has a wave of its own
    static_assert(kPrepThreads == 512, "the block assignment is for eight waves");
    for (int nb = 0; nb < (wave < 2 ? 2 : 1); ++nb) {
        // blk -> (i, jb): 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) ...
        // wave 0: blocks 0, 9; wave 1: 2, 5; waves 2..7: 1, 3, 4, 6, 7, 8
        const int blk = wave == 0 ? 9 * nb
                      : wave == 1 ? 2 + 3 * nb
                      : wave == 2 ? 1 : wave < 5 ? wave : wave + 1;
        const int i = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
        const int jb = blk - (i * (i + 1)) / 2;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 32 * ks + 8 * b;
            const bf16x8 ar = lds8_rq(sm.KR, 16 * i + m, 4 * ks + b);
            const bf16x8 aq = lds8_rq(sm.QR, 16 * i + m, 4 * ks + b);
            bf16x8 bc = lds8_rq(sm.KCD, 16 * jb + m, 4 * ks + b);
            if (jb < i) {
                const float *f = &sm.F[pair_index(i, jb)][ch];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    bc[e] = (bf16)((float)bc[e] * f[e]);
            }
            accA = mfma16(ar, bc, accA);
            accP = mfma16(aq, bc, accP);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int row = 16 * i + 4 * b + e, col = 16 * jb + m;
            sm.AM[row][col] = (jb < i || col < row) ? sm.AM[row][kChunk] * accA[e] : 0.f;
            sm.PM[row][col] = (bf16)((jb < i || col <= row) ? scale * accP[e] : 0.f);
        }
    }
    __syncthreads();

    if (load_next)
        prep_load_token(in, q, k, v, g, beta, next, H, wave, tg, cq, 1);
    // ---- phase 3: T = (I + A)^-1 ------------------------------------------------
    if (wave == 0) {
        // diagonal 16 x 16 blocks by forward substitution, one column per lane;
        // x[s] = 0 for s < col, so the full-range sums only add zeros there
        // (column form: once x[s] is final it updates every later row at once,
        // so the dependency depth is 16 instead of 120)
        // the start vector depends only on the lane: made opaque here, so the
        // compiler forms it per chunk instead of holding 16 registers (or
        // spill slots) through the whole persistent loop
        int col = lane & 15;
        asm volatile("" : "+v"(col));
        const int blk = lane >> 4, o = 16 * blk;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            x[r] = (r == col) ? 1.f : 0.f;
#pragma unroll
        for (int s2 = 0; s2 < 15; ++s2)
#pragma unroll
            for (int r = s2 + 1; r < 16; ++r)
                x[r] -= sm.AM[o + r][o + s2] * x[s2];
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ts.TM[o + r][o + col] = x[r];
    } else if (wave <= 2) {
        // T_01 and T_23 are read by the W / U~ products: zero them
        const int o = (wave == 1) ? 0 : 32;
#pragma unroll
        for (int e = lane; e < 256; e += 64)
            ts.TM[o + e / 16][o + 16 + e % 16] = 0.f;
    }
    __syncthreads();
    // off-diagonal blocks by distance on fp32 MFMA (16x16x4), one block per wave:
    // X = sum_{mm=bb}^{a-1} A_a,mm T_mm,bb ;  T_a,bb = -T_aa X
    for (int dist = 1; dist < 4; ++dist) {
        if (wave < 4 - dist) {
            const int a = wave + dist, bb = wave;
            f32x4 X = {0.f, 0.f, 0.f, 0.f};
            for (int mm = bb; mm < a; ++mm) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk)
                    X = mfma4_f32(sm.AM[16 * a + m][16 * mm + 4 * kk + b],
                                  ts.TM[16 * mm + 4 * kk + b][16 * bb + m], X);
            }
            // k order: MFMA kk takes k = 4 b + kk, which is X's own accumulator row
            f32x4 Y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < 4; ++kk)
                Y = mfma4_f32(ts.TM[16 * a + m][16 * a + 4 * b + kk], X[kk], Y);
#pragma unroll
            for (int i = 0; i < 4; ++i)
                ts.TM[16 * a + 4 * b + i][16 * bb + m] = -Y[i];
        }
        // wave bb reads and writes only column bb of T (besides the diagonal
        // blocks, final since the barrier above), so only the last distance
        // needs the workgroup barrier, before phase 4 reads all of T
        wave_or_group_sync(dist == 3);
    }

    if (load_next)
        prep_load_token(in, q, k, v, g, beta, next, H, wave, tg, cq, 2);
    // ---- phase 4: W = T X and U~ = T V for the wave's 16 channels --------------
    // (kBwd) dY and Z of token tid / 8, channels 16 (tid % 8) .. + 15, for dO
    bf16x8 dyb[2], zb[2];
    if constexpr (kBwd) {
        const int r = tid >> 3, cb = 16 * (tid & 7);
        const int64_t off = ((pt.tok0 + (r < pt.len ? r : pt.len - 1)) * H + pt.h) * (int64_t)kDV + cb;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            dyb[p] = *reinterpret_cast<const bf16x8 *>(bo.dout + off + 8 * p);
            zb[p] = *reinterpret_cast<const bf16x8 *>(bo.gate + off + 8 * p);
        }
    }
    const int nt = wave;                       // channels 16 nt .. 16 nt + 15
    f32x4 accW[4], accU[4];
    {
        bf16x8 tf[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 f = {};
                if (ks <= (mt >> 1)) {
                    const float *t = &ts.TM[16 * mt + m][32 * ks + 8 * b];
                    const f32x4 lo = *reinterpret_cast<const f32x4 *>(t);
                    const f32x4 hi = *reinterpret_cast<const f32x4 *>(t + 4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f[e] = (bf16)lo[e];
                        f[4 + e] = (bf16)hi[e];
                    }
                }
                tf[mt][ks] = f;
            }
        bf16x8 xf[2], vf[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            xf[ks] = lds8(&sm.XB[16 * nt + m][32 * ks + 8 * b]);
            vf[ks] = lds8(&sm.VB[16 * nt + m][32 * ks + 8 * b]);
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            accW[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            accU[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                if (ks <= (mt >> 1)) {
                    accW[mt] = mfma16(tf[mt][ks], xf[ks], accW[mt]);
                    accU[mt] = mfma16(tf[mt][ks], vf[ks], accU[mt]);
                }
        }
        if constexpr (kExt) {
            // per-chunk records also keep W and U~ as row fragments for the
            // gradient kernel: the transposed products X^T T^T = W^T and
            // V^T T^T = U~^T leave the wave's 16 channels of one token row as
            // four consecutive k of the row's fragment (half of a 16-byte slot)
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 wt = {0.f, 0.f, 0.f, 0.f}, ut = wt;
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    if (ks <= (mt >> 1)) {
                        wt = mfma16(xf[ks], tf[mt][ks], wt);
                        ut = mfma16(vf[ks], tf[mt][ks], ut);
                    }
                const size_t off = (mt * 4 + (nt >> 1)) * kFragBytes + lane * 16 + (nt & 1) * 8;
                *reinterpret_cast<bf16x4 *>(rec + kOffXW + off) = to_bf16x4(wt, 1.f);
                *reinterpret_cast<bf16x4 *>(rec + kOffXU + off) = to_bf16x4(ut, 1.f);
            }
        }
    }

    if (load_next)
        prep_load_token(in, q, k, v, g, beta, next, H, wave, tg, cq, 3);
    // (kBwd) dO^T = (dY sigmoid(Z))^T [dv][token] in KCD's space (free since phase
    // 2); the 8-token group of row c sits at group ^ ((c >> 4) & 7), so that the
    // rows 16 apart that one wave writes at once fall in different LDS banks
    bf16 (*const dot)[kColLd] = reinterpret_cast<bf16 (*)[kColLd]>(&sm.KCD[0][0]);
    if constexpr (kBwd) {
        const int r = tid >> 3, cb = 16 * (tid & 7);
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = cb + 8 * p + e;
                const float x = r < pt.len ? (float)dyb[p][e] * sigmoidf_((float)zb[p][e]) : 0.f;
                dot[c][8 * ((r >> 3) ^ ((c >> 4) & 7)) + (r & 7)] = (bf16)x;
            }
        __syncthreads();
    }
    if constexpr (kMode == 2) {
        // every wave is past phase 4: the A / T, X and V tiles are free for the
        // composition operands below
        __syncthreads();
    }
    // ---- phase 5: L, Bm, Q^, O0 for the wave's 16 channels ----------------------
    {
        bf16x8 wf[2], uf[2];                   // W^T as A operand, U~ as B operand (perm k)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            wf[ks] = acc_to_frag(accW[2 * ks], accW[2 * ks + 1]);
            uf[ks] = acc_to_frag(accU[2 * ks], accU[2 * ks + 1]);
        }
        const int half = nt & 1, kq = nt >> 1;  // fragment half and dk k-step of these channels
        if constexpr (kMode == 0) {
            // L^T rows 16 nt.. = W^T K'  ->  -L fragments (mt, kq), elements 4 half .. 4 half + 3
            // Bm columns 16 nt.. = K'^T U~ ->  Bm of value block nt; row tiles 2 mp and
            // 2 mp + 1 fill one 16-byte slot per lane, stored with one instruction
    #pragma unroll
            for (int mp = 0; mp < 4; ++mp) {
                f32x4 bmv[2];
    #pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int mt = 2 * mp + s2;
                    bf16x8 kpf[2];
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        kpf[ks] = perm8(&sm.KPT[16 * mt + m][0], ks, b);
                    f32x4 l = {0.f, 0.f, 0.f, 0.f}, bm = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        l = mfma16(wf[ks], kpf[ks], l);
                        bm = mfma16(kpf[ks], uf[ks], bm);
                    }
                    if constexpr (kBwd) {
                        // -L^T fragment (row tile nt, k-step mt / 2), elements
                        // 4 (mt % 2) .. + 3: the same bf16 values as the -L stored
                        // above, transposed exactly (a product with the identity)
                        bf16x4 id;
    #pragma unroll
                        for (int e = 0; e < 4; ++e)
                            id[e] = (bf16)(4 * b + e == m ? 1.f : 0.f);
                        const f32x4 tr = mfma16k16(to_bf16x4(l, -1.f), id, f32x4{0.f, 0.f, 0.f, 0.f});
                        *reinterpret_cast<bf16x4 *>(bo.rec + kOffLN + (nt * 4 + (mt >> 1)) * kFragBytes +
                                                    lane * 16 + (mt & 1) * 8) = to_bf16x4(tr, 1.f);
                    }
                    *reinterpret_cast<bf16x4 *>(rec + kOffLN + (mt * 4 + kq) * kFragBytes +
                                                lane * 16 + half * 8) = to_bf16x4(l, -1.f);
                    bmv[s2] = bm;
                }
                const bf16x4 b0 = to_bf16x4(bmv[0], 1.f), b1 = to_bf16x4(bmv[1], 1.f);
                *reinterpret_cast<bf16x8 *>(rec + kOffBM + nt * 4096 + mp * 1024 + lane * 16) =
                    bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            }
        }
        if constexpr (kMode <= 1) {
            // Q^ = scale Q e^G - P W  (as Q^^T rows 16 nt..)  and  O0 = P U~ for value block nt;
            // O0 row tiles 2 tp and 2 tp + 1 share one 16-byte slot per lane
    #pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                f32x4 o0v[2];
    #pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int mt = 2 * tp + s2;
                    // P is lower triangular: token tiles 0 and 1 have no columns in k-step 1
                    bf16x8 pf[2];
    #pragma unroll
                    for (int ks = 0; ks <= (mt >> 1); ++ks)
                        pf[ks] = perm8(&sm.PM[16 * mt + m][0], ks, b);
                    // scale Q e^G at row 16 mt + m, channels 16 nt + 4 b .. + 3, from q e^{G - B_mt}
                    const bf16x4 qr =
                        *reinterpret_cast<const bf16x4 *>(&sm.QR[16 * mt + m][rq(16 * mt + m, 4 * nt + b)]);
                    const f32x4 eb = *reinterpret_cast<const f32x4 *>(&sm.eB[mt][16 * nt + 4 * b]);
                    f32x4 qh;
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
                        qh[i] = -scale * (float)qr[i] * eb[i];
                    f32x4 o0 = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll
                    for (int ks = 0; ks <= (mt >> 1); ++ks) {
                        qh = mfma16(wf[ks], pf[ks], qh);   // (P W)^T - (scale Q e^G)^T
                        o0 = mfma16(uf[ks], pf[ks], o0);   // (P U~)^T
                    }
                    *reinterpret_cast<bf16x4 *>(rec + kOffQH + (mt * 4 + kq) * kFragBytes +
                                                lane * 16 + half * 8) = to_bf16x4(qh, -1.f);
                    if constexpr (kBwd) {
                        // Q^^T [dk][token] in XB's space (free since phase 4)
                        const bf16x4 qv = to_bf16x4(qh, -1.f);
    #pragma unroll
                        for (int i = 0; i < 4; ++i)
                            sm.XB[16 * nt + 4 * b + i][16 * mt + m] = qv[i];
                    }
                    o0v[s2] = o0;
                }
                const bf16x4 a0 = to_bf16x4(o0v[0], 1.f), a1 = to_bf16x4(o0v[1], 1.f);
                *reinterpret_cast<bf16x8 *>(rec + kOffO0 + nt * 2048 + tp * 1024 + lane * 16) =
                    bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            }
        }
        if constexpr (kBwd) {
            // Q^^T dO for value block nt, in the record's Bm layout (fragment i2
            // holds dk row tiles 2 i2 and 2 i2 + 1), from the Q^^T and dO^T tiles
            __syncthreads();
#pragma unroll
            for (int i2 = 0; i2 < 4; ++i2) {
                f32x4 acc[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int t = 2 * i2 + s2;
                    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        a = mfma16(lds8(&sm.XB[16 * t + m][32 * ks + 8 * b]),
                                   lds8(&dot[16 * nt + m][8 * ((4 * ks + b) ^ nt)]), a);
                    acc[s2] = a;
                }
                *reinterpret_cast<bf16x8 *>(bo.rec + kOffBM + nt * 4096 + i2 * 1024 + lane * 16) =
                    acc_to_frag(acc[0], acc[1]);
            }
        }
        if constexpr (kExt) {
            // T^T and P^T, eight elements of one row per thread (T below its
            // diagonal blocks only: the tiles above them are not all written)
            const int r = tid >> 3, s0 = 8 * (tid & 7);
            bf16x8 tt, pt8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int s = s0 + e;
                tt[e] = (bf16)(s >= r ? ts.TM[s][r] : 0.f);
                pt8[e] = sm.PM[s][r];
            }
            *reinterpret_cast<bf16x8 *>(rec + kOffXT + (size_t)(r * kChunk + s0) * 2) = tt;
            *reinterpret_cast<bf16x8 *>(rec + kOffXP + (size_t)(r * kChunk + s0) * 2) = pt8;
        }
        if constexpr (kMode == 1) {
            // -L0 and Bm0 with rows on the k index: L0 block (mt, nt) as K'^T W with
            // K'^T as the A operand, so tiles 2 ks and 2 ks + 1 form k-step ks
#pragma unroll
            for (int ks2 = 0; ks2 < 4; ++ks2) {
                f32x4 lc[2], bc[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int mt = 2 * ks2 + s2;
                    bf16x8 kpf[2];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        kpf[ks] = perm8(&sm.KPT[16 * mt + m][0], ks, b);
                    lc[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
                    bc[s2] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks) {
                        lc[s2] = mfma16(kpf[ks], wf[ks], lc[s2]);   // L0[16 mt + 4 b + i][16 nt + m]
                        bc[s2] = mfma16(kpf[ks], uf[ks], bc[s2]);   // Bm0, same place
                    }
                }
                hold.nl0[ks2] = acc_to_frag(-lc[0], -lc[1]);
                hold.bm0[ks2] = acc_to_frag(bc[0], bc[1]);
            }
        }
        if constexpr (kMode == 2) {
            // M1 = D1 - L1 and Q^1 as A fragments (the record's LN / QH layouts) in
            // LDS, each wave writing its 16 columns; the fp32 terms -L1 D0 and
            // Q^1 D0 stay in registers, Bm1 and O0_1 are formed after the barrier
            bf16x8 *m1s = reinterpret_cast<bf16x8 *>(&sm.KR[0][0]);   // [32 fragments][64 lanes]
            bf16x8 *q1s = reinterpret_cast<bf16x8 *>(&sm.XB[0][0]);   // [16 fragments][64 lanes]
            const f32x4 d0c = *reinterpret_cast<const f32x4 *>(&sm.DEC0[16 * nt + 4 * b]);
            const float d1 = sm.eGB[0][16 * nt + m];                  // e^{G_end} of chunk 1
            f32x4 nld[8], qd[4];
#pragma unroll
            for (int mt = 0; mt < 8; ++mt) {
                bf16x8 kpf[2];
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    kpf[ks] = perm8(&sm.KPT[16 * mt + m][0], ks, b);
                f32x4 l = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks)
                    l = mfma16(wf[ks], kpf[ks], l);       // L1[16 mt + m][16 nt + 4 b + i]
                f32x4 mm;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    mm[i] = (mt == nt && m == 4 * b + i) ? d1 - l[i] : -l[i];
                    nld[mt][i] = -l[i] * d0c[i];
                }
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint8_t *>(&m1s[(mt * 4 + kq) * 64 + lane]) +
                                            8 * half) = to_bf16x4(mm, 1.f);
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                bf16x8 pf[2];
#pragma unroll
                for (int ks = 0; ks <= (tt >> 1); ++ks)
                    pf[ks] = perm8(&sm.PM[16 * tt + m][0], ks, b);
                const bf16x4 qr =
                    *reinterpret_cast<const bf16x4 *>(&sm.QR[16 * tt + m][rq(16 * tt + m, 4 * nt + b)]);
                const f32x4 eb = *reinterpret_cast<const f32x4 *>(&sm.eB[tt][16 * nt + 4 * b]);
                f32x4 qh;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    qh[i] = -scale * (float)qr[i] * eb[i];
#pragma unroll
                for (int ks = 0; ks <= (tt >> 1); ++ks)
                    qh = mfma16(wf[ks], pf[ks], qh);      // -Q^1[16 tt + m][16 nt + 4 b + i]
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    qd[tt][i] = -qh[i] * d0c[i];
                *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint8_t *>(&q1s[(tt * 4 + kq) * 64 + lane]) +
                                            8 * half) = to_bf16x4(qh, -1.f);
            }
            __syncthreads();
            // -L01 = -L1 D0 + M1 (-L0) and Bm01 = Bm1 + M1 Bm0 for the wave's columns
#pragma unroll
            for (int mp = 0; mp < 4; ++mp) {
                f32x4 bmv[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int mt = 2 * mp + s2;
                    bf16x8 kpf[2];
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        kpf[ks] = perm8(&sm.KPT[16 * mt + m][0], ks, b);
                    f32x4 accl = nld[mt], accb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < 2; ++ks)
                        accb = mfma16(kpf[ks], uf[ks], accb);    // Bm1[16 mt + 4 b + i][16 nt + m]
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 mf = m1s[(mt * 4 + ks) * 64 + lane];
                        accl = mfma16(hold.nl0[ks], mf, accl);   // rows 16 mt + m, cols 16 nt + 4 b + i
                        accb = mfma16(mf, hold.bm0[ks], accb);   // rows 16 mt + 4 b + i, col 16 nt + m
                    }
                    *reinterpret_cast<bf16x4 *>(rec + kOffLN + (mt * 4 + kq) * kFragBytes +
                                                lane * 16 + half * 8) = to_bf16x4(accl, 1.f);
                    bmv[s2] = accb;
                }
                const bf16x4 b0 = to_bf16x4(bmv[0], 1.f), b1 = to_bf16x4(bmv[1], 1.f);
                *reinterpret_cast<bf16x8 *>(rec + kOffBM + nt * 4096 + mp * 1024 + lane * 16) =
                    bf16x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
            }
            // Q^1' = Q^1 D0 + Q^1 (-L0) and O0_1' = O0_1 + Q^1 Bm0
#pragma unroll
            for (int tp = 0; tp < 2; ++tp) {
                f32x4 o0v[2];
#pragma unroll
                for (int s2 = 0; s2 < 2; ++s2) {
                    const int tt = 2 * tp + s2;
                    bf16x8 pf[2];
#pragma unroll
                    for (int ks = 0; ks <= (tt >> 1); ++ks)
                        pf[ks] = perm8(&sm.PM[16 * tt + m][0], ks, b);
                    f32x4 accq = qd[tt], acco = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks <= (tt >> 1); ++ks)
                        acco = mfma16(uf[ks], pf[ks], acco);     // O0_1[16 tt + m][16 nt + 4 b + i]
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks) {
                        const bf16x8 qf = q1s[(tt * 4 + ks) * 64 + lane];
                        accq = mfma16(hold.nl0[ks], qf, accq);   // rows 16 tt + m, cols 16 nt + 4 b + i
                        acco = mfma16(hold.bm0[ks], qf, acco);
                    }
                    *reinterpret_cast<bf16x4 *>(rec + kOffQH1 + (tt * 4 + kq) * kFragBytes +
                                                lane * 16 + half * 8) = to_bf16x4(accq, 1.f);
                    o0v[s2] = acco;
                }
                const bf16x4 a0 = to_bf16x4(o0v[0], 1.f), a1 = to_bf16x4(o0v[1], 1.f);
                *reinterpret_cast<bf16x8 *>(rec + kOffO01 + nt * 2048 + tp * 1024 + lane * 16) =
                    bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            }
        }
    }
    // the next chunk's phase 1 rewrites the LDS operands
    __syncthreads();
}

// Chunk 0 and chunk 1 (valid = false when the sequence ends first) of pair
// task t = pair slot * H + h; c0.valid = false for a padding slot.
__device__ __forceinline__ void pair_tasks(const int32_t *cu, int N, int T, int H, int64_t t,
                                           PrepTask &c0, PrepTask &c1)
{
    const int64_t slot = t / H;
    c0 = PrepTask{};
    c1 = PrepTask{};
    c0.h = c1.h = (int)(t % H);
    c0.rec = c1.rec = t;
    int n;
    int64_t j;
    if (!slot_to_step<kPairTokens>(cu, N, T, slot, n, j))
        return;
    const SeqInfo si = seq_info(cu, n, T, kPairTokens);
    const int64_t rem = si.len - j * kPairTokens;
    const int plen = rem < kPairTokens ? (int)rem : kPairTokens;
    c0.valid = true;
    c0.tok0 = si.bos + j * kPairTokens;
    c0.len = plen < kChunk ? plen : kChunk;
    if (plen > kChunk) {
        c1.valid = true;
        c1.tok0 = c0.tok0 + kChunk;
        c1.len = plen - kChunk;
    }
}

// The prep kernel is persistent: workgroup b handles tasks b, b + G, b + 2 G,
// ... (G = grid size, a multiple of 8 so that with H a multiple of 8 every
// task of head h runs on XCD h % 8, where the chain walks head h).  The inputs
// of the next chunk are loaded into registers while the current one is in its
// matrix phases, so only the first chunk of a workgroup waits for memory.
// kPair: a task is a pair of chunks (see kPairRecBytes), else one chunk.
// kBwd (per-chunk records only): also every chunk's backward record in ws_b,
// from the gate logits and dY.
template <bool kPro, bool kPair, bool kBwd = false>
__global__ __launch_bounds__(kPrepThreads) void kda_prep_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, const int32_t *__restrict__ cu,
    int N, int T, int H, int64_t n_tasks, float scale, unsigned pro, uint8_t *__restrict__ ws,
    const bf16 *__restrict__ gate, const bf16 *__restrict__ dout, uint8_t *__restrict__ ws_b)
{
    static_assert(!kBwd || (!kPair && !kPro), "the fused backward record needs per-chunk records");
    extern __shared__ __align__(16) uint8_t smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    TSmem &ts = *reinterpret_cast<TSmem *>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int tg = lane & 15, cq = lane >> 4;
    PairHold hold;
    PrepIn in;
    int64_t t = blockIdx.x;
    if constexpr (!kPair) {
        PrepTask next = t < n_tasks ? prep_task(cu, N, T, H, t) : PrepTask{};
        if (t < n_tasks && next.valid)
            prep_load(in, q, k, v, g, beta, next, H, wave, tg, cq);
        for (; t < n_tasks; t += gridDim.x) {
            const PrepTask pt = next;
            const int64_t tn = t + gridDim.x;
            if (tn < n_tasks)
                next = prep_task(cu, N, T, H, tn);
            const bool load_next = tn < n_tasks && next.valid;
            if (!pt.valid) {
                if (load_next)
                    prep_load(in, q, k, v, g, beta, next, H, wave, tg, cq);
                continue;
            }
            prep_chunk<kPro, 0, true, kBwd>(
                sm, ts, in, q, k, v, g, beta, pt, next, load_next, H, scale, pro,
                ws + pt.rec * (int64_t)kChunkRecBytes, hold,
                BwdOut{gate, dout, kBwd ? ws_b + pt.brec * (int64_t)kChunkRecBytes : nullptr});
        }
    } else {
        PrepTask c0, c1;
        if (t < n_tasks)
            pair_tasks(cu, N, T, H, t, c0, c1);
        else
            c0 = c1 = PrepTask{};
        if (t < n_tasks && c0.valid)
            prep_load(in, q, k, v, g, beta, c0, H, wave, tg, cq);
        for (; t < n_tasks; t += gridDim.x) {
            const PrepTask p0 = c0, p1 = c1;
            const int64_t tn = t + gridDim.x;
            if (tn < n_tasks)
                pair_tasks(cu, N, T, H, tn, c0, c1);
            else
                c0 = c1 = PrepTask{};
            if (!p0.valid) {
                if (c0.valid)
                    prep_load(in, q, k, v, g, beta, c0, H, wave, tg, cq);
                continue;
            }
            uint8_t *rec = ws + p0.rec * (int64_t)kPairRecBytes;
            if (p1.valid) {
                prep_chunk<kPro, 1>(sm, ts, in, q, k, v, g, beta, p0, p1, true, H, scale, pro, rec,
                                    hold);
                prep_chunk<kPro, 2>(sm, ts, in, q, k, v, g, beta, p1, c0, c0.valid, H, scale, pro,
                                    rec, hold);
            } else {
                prep_chunk<kPro, 0>(sm, ts, in, q, k, v, g, beta, p0, c0, c0.valid, H, scale, pro,
                                    rec, hold);
            }
        }
    }
}

namespace {

// Chain workgroup: 8 compute waves and 1 store wave.  Compute wave w keeps
// state rows 16 w .. 16 w + 15 (one 16-row tile) and applies
// S' = dec S + Bm - L S chunk after chunk; the waves exchange the new state as
// bf16 MFMA fragments through LDS.  The step is bound by the CU's vector
// memory pipeline, which costs about the same per load instruction whatever
// its width: so the compute waves load only their 16-byte-per-lane fragments
// of L, and a side wave fetches this value block's Bm and the decay vector
// (5 wide loads instead of 16 narrow ones) two chunks ahead into an LDS ring.
// The store wave copies each chunk's entry state from LDS to the workspace for
// the output kernel.  Only the store wave issues stores: the loading waves
// (compute and side) can then wait for exactly the loads they need.  Keeping loads and stores in different
// waves lets the compiler wait for exactly the prefetched stage it needs
// (with both kinds pending it can only wait for everything).
constexpr int kComputeWaves = 8;
constexpr int kStoreWave = kComputeWaves;
constexpr int kSideWave = kComputeWaves + 1;
// with kNB value blocks per workgroup (see the kernel), side waves of at most
// two blocks each
template <int kNB> constexpr int chain_side_waves() { return kNB <= 2 ? 1 : kNB / 2; }
template <int kNB> constexpr int chain_threads() { return 64 * (kComputeWaves + 1 + chain_side_waves<kNB>()); }
// Chunks of operands in flight per compute wave (L) and per side wave (Bm,
// dec).  Records in HBM (a long sequence) make a step about half again as
// long as records still in the last-level cache, and deeper prefetch does not
// shorten it: the step is then bound by the loads and stores one CU keeps in
// flight, not by the latency of one load.
constexpr int kPrefetch = 4;
constexpr int kSideSets = kPrefetch;

// the second chain of a launch that runs two (ws null: none)
struct ChainJob2 {
    const float *init;
    float *final_state;
    uint8_t *ws;
    int wgs;        // workgroups of the first chain
};

struct ChainStage {
    bf16x8 ln[4];      // -L rows of the wave's state tile, 4 dk k-steps
};

__device__ __forceinline__ void chain_load(ChainStage &st, const uint8_t *rec_any, int w,
                                           int lane)
{
    const gbyte *rec = uniform_gptr(rec_any);    // the record base is the same for the wave
    const uint32_t lo = (uint32_t)lane * 16u;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        st.ln[ks] = gload<bf16x8>(rec, kOffLN + (w * 4 + ks) * kFragBytes + lo);
}

}  // namespace

// With kSnap the chain also writes fp32 state snapshots every snap_steps
// steps (see snap_slot0): the compute waves park the state in LDS at a
// snapshot boundary and the store wave writes it out in the next iteration, so
// the compute waves still issue no stores inside the loop.
//
// kNB value blocks per workgroup (1, 2 or 4; kNB > 1 only without snapshots):
// the waves apply every step to kNB adjacent 16-column blocks with the same L
// fragments, so a (sequence, head) takes 8 / kNB workgroups, which stream L
// once for kNB blocks.  Each side wave fetches Bm for two blocks at most.
//
// kPair: the records are pair records (kPairRecBytes), one step per pair of
// chunks; the step's arithmetic is the same.
//
// job2 (ws not null, no snapshots): a second chain over other records of the
// same shape runs in workgroups job2.wgs .. 2 job2.wgs - 1 of the launch, with
// its own initial and final state.
template <bool kSnap, int kNB = 1, bool kPair = false>
__global__ __launch_bounds__(chain_threads<kNB>()) void kda_chain_bf16_kernel(
    const float *__restrict__ init, float *__restrict__ final_state, float *__restrict__ snaps,
    int snap_steps, const int32_t *__restrict__ cu, int T, int H, int units,
    uint8_t *__restrict__ ws, ChainJob2 job2)
{
    constexpr int kStep = kPair ? kPairTokens : kChunk;           // tokens per step
    constexpr size_t kRec = kPair ? kPairRecBytes : kChunkRecBytes;    // record stride
    static_assert(kNB == 1 || kNB == 2 || kNB == 4, "1, 2 or 4 value blocks per workgroup");
    static_assert(!kSnap || kNB == 1, "snapshots with one value block per workgroup");
    constexpr int kSideBlocks = kNB == 1 ? 1 : 2;   // value blocks per side wave
    // state as 4 k-step fragments per value block; wave w writes elements
    // 4 (w % 2) .. + 3 of k-step w / 2
    __shared__ bf16x8 sbuf[2][kNB][4][64];
    // Bm of these value blocks (the record's fragment layout) and dec, per
    // chunk, in a 2-slot ring: slot j & 1 holds chunk j
    __shared__ bf16x8 side_bm[2][kNB][4][64];
    __shared__ float side_dec[2][kDK];
    __shared__ float snap_s[kSnap ? 2 : 1][kSnap ? kDK : 1][kVBlock];

    // all value blocks of one (sequence, head) land on the same XCD (blocks are
    // dealt to the 8 XCDs round-robin), so they share that XCD's L2
    constexpr int kWgPerUnit = kNumVBlocks / kNB;
    int id = blockIdx.x;
    if (!kSnap && job2.ws && id >= job2.wgs) {
        id -= job2.wgs;
        init = job2.init;
        final_state = job2.final_state;
        ws = job2.ws;
    }
    const int xcd = id & 7, qid = id >> 3;
    const int unit = (int)((unsigned)qid / kWgPerUnit) * 8 + xcd;
    const int blk = (int)((unsigned)qid % kWgPerUnit) * kNB;   // first value block of the workgroup
    if (unit >= units)
        return;
    const int n = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
    const int m = lane & 15, b = lane >> 4;
    const SeqInfo si = seq_info(cu, n, T, kStep);
    const int64_t nch = (si.len + kStep - 1) / kStep;             // steps of the sequence
    auto rec_of = [&](int64_t jc) { return ws + ((si.slot0 + jc) * H + h) * (int64_t)kRec; };
    // a snapshot is due on entry to step jb (after jb full steps)
    auto snap_at = [&](int64_t jb) {
        return kSnap && jb >= 1 && jb <= nch && jb % snap_steps == 0 && jb * kStep <= si.len;
    };

    // the chunk loop runs in rounds of kPrefetch iterations; iterations past the
    // last chunk (at most kPrefetch - 1) leave the state unchanged
    const int64_t niter = (nch + kPrefetch - 1) / kPrefetch * kPrefetch;
    if (chain_side_waves<kNB>() == 1 ? w == kSideWave : w >= kSideWave) {
        // side operands of chunk jc (past the end: the last chunk) into register
        // set jc % kSideSets, later into ring slot jc & 1: a chunk's loads are
        // issued kSideSets steps before it is staged, so each wait leaves the
        // newer sets' loads in flight (on a long sequence the records come
        // from HBM, whose latency spans several steps).  Side wave sw fetches
        // Bm of blocks sw * kSideBlocks .. + kSideBlocks - 1 (of the
        // workgroup's), and side wave 0 the decay vector too.
        constexpr bool kOneSide = chain_side_waves<kNB>() == 1;
        const int sb0 = kOneSide ? 0 : (w - kSideWave) * kSideBlocks;
        bf16x8 nbm[kSideSets][kSideBlocks][4];
        f32x2 ndec[kSideSets];
        auto side_load = [&](int set, int64_t jc) {
            const gbyte *rec = uniform_gptr(rec_of(jc < nch ? jc : nch - 1));
#pragma unroll
            for (int vb = 0; vb < kSideBlocks; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    nbm[set][vb][i] = gload<bf16x8>(
                        rec, kOffBM + (blk + sb0 + vb) * 4096 + i * 1024 + lane * 16u);
            if (kOneSide || sb0 == 0)
                ndec[set] = gload<f32x2>(rec, kOffDEC + lane * 8u);
        };
        auto side_store = [&](int set, int slot) {
#pragma unroll
            for (int vb = 0; vb < kSideBlocks; ++vb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    side_bm[slot][sb0 + vb][i][lane] = nbm[set][vb][i];
            if (kOneSide || sb0 == 0)
                *reinterpret_cast<f32x2 *>(&side_dec[slot][2 * lane]) = ndec[set];
        };
        if (nch > 0) {
            side_load(0, 0);
            side_store(0, 0);
#pragma unroll
            for (int c = 1; c <= kSideSets; ++c)
                side_load(c % kSideSets, c);
        }
        __syncthreads();
        // niter is a multiple of kSideSets; in step jc stage chunk jc + 1, read
        // in the next step, and refill its set with chunk jc + 1 + kSideSets
        for (int64_t j0 = 0; j0 < niter; j0 += kSideSets) {
#pragma unroll
            for (int s = 0; s < kSideSets; ++s) {
                const int set = (s + 1) % kSideSets;
                side_store(set, (int)((j0 + s + 1) & 1));
                side_load(set, j0 + s + 1 + kSideSets);
                __syncthreads();
            }
        }
        return;
    }
    if (w == kStoreWave) {
        // snapshot jb: rows 16 i + lane / 4, channels 16 blk + 4 (lane % 4) .. + 3
        auto write_snap = [&](int64_t jb) {
            const int64_t slot =
                snap_slot0(cu, n, T, snap_steps * kStep) + jb / snap_steps - 1;
            float *dst = snaps + (slot * H + h) * (int64_t)(kDK * kDV) + kVBlock * blk +
                         4 * (lane & 3);
#pragma unroll
            for (int i = 0; i < kDK / 16; ++i) {
                const int row = 16 * i + (lane >> 2);
                *reinterpret_cast<f32x4 *>(dst + row * kDV) =
                    *reinterpret_cast<const f32x4 *>(&snap_s[jb & 1][row][4 * (lane & 3)]);
            }
        };
        // store wave: copy the entry state of chunk jc (4 fragments, 16 B per lane each)
        __syncthreads();
        for (int64_t jc = 0; jc < niter; ++jc) {
            if (jc < nch) {
#pragma unroll
                for (int vb = 0; vb < kNB; ++vb) {
                    bf16x8 *dst =
                        reinterpret_cast<bf16x8 *>(rec_of(jc) + kOffSB + (blk + vb) * 4096) + lane;
#pragma unroll
                    for (int ks = 0; ks < 4; ++ks)
                        dst[ks * 64] = sbuf[jc & 1][vb][ks][lane];
                }
            }
            if constexpr (kSnap) {
                if (snap_at(jc))
                    write_snap(jc);
            }
            __syncthreads();
        }
        if constexpr (kSnap) {
            if (snap_at(niter))
                write_snap(niter);
        }
        return;
    }

    const int64_t sbase = (int64_t)unit * (kDK * kDV);
    const int col = kVBlock * blk + m;         // column in the first block (+16 per block)
    const int row0 = 16 * w + 4 * b;           // the wave's rows row0 + i, column col
    // this wave's half of k-step fragment w / 2 of block vb, as 4 bf16 at byte
    // 8 (w % 2) of a lane's slot
    auto put_state = [&](int buf, int vb, const f32x4 &x) {
        *reinterpret_cast<bf16x4 *>(reinterpret_cast<uint8_t *>(&sbuf[buf][vb][w >> 1][lane]) +
                                    8 * (w & 1)) = bf16x4{(bf16)x[0], (bf16)x[1], (bf16)x[2],
                                                          (bf16)x[3]};
    };
    f32x4 S[kNB];
#pragma unroll
    for (int vb = 0; vb < kNB; ++vb) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[vb][i] = init ? init[sbase + (row0 + i) * kDV + col + kVBlock * vb] : 0.f;
        put_state(0, vb, S[vb]);
    }
    __syncthreads();

    // the scheduling barriers keep each stage's loads together and in stage
    // order, in the prologue and in the loop alike, so the loop-entry wait
    // state is the same on both paths and every wait stays partial; stage
    // loads past the last chunk re-read the last chunk so that every iteration
    // issues the same loads
    auto load_stage = [&](ChainStage &stage, int64_t jc) {
        const int64_t jl = jc < nch ? jc : nch - 1;
        __builtin_amdgcn_sched_barrier(0);
        chain_load(stage, rec_of(jl), w, lane);
        __builtin_amdgcn_sched_barrier(0);
    };
    ChainStage st[kPrefetch];
    if (nch > 0) {
#pragma unroll
        for (int s = 0; s < kPrefetch; ++s)
            load_stage(st[s], s);
    }

    for (int64_t j0 = 0; j0 < niter; j0 += kPrefetch) {
#pragma unroll
        for (int s = 0; s < kPrefetch; ++s) {
            const int64_t jc = j0 + s;
            const ChainStage &c = st[s];
            const f32x4 dec = *reinterpret_cast<const f32x4 *>(&side_dec[jc & 1][row0]);
#pragma unroll
            for (int vb = 0; vb < kNB; ++vb) {
                const bf16x8 *sb = &sbuf[jc & 1][vb][0][lane];
                const bf16x4 bm = *reinterpret_cast<const bf16x4 *>(
                    reinterpret_cast<const uint8_t *>(&side_bm[jc & 1][vb][w >> 1][lane]) +
                    8 * (w & 1));
                // S' = dec S + Bm - L S for the wave's 16 rows
                f32x4 acc;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[i] = dec[i] * S[vb][i] + (float)bm[i];
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    acc = mfma16(c.ln[ks], sb[ks * 64], acc);
                if (jc < nch)
                    S[vb] = acc;
                put_state((jc + 1) & 1, vb, S[vb]);
            }
            if constexpr (kSnap) {
                if (snap_at(jc + 1)) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        snap_s[(jc + 1) & 1][row0 + i][m] = S[0][i];
                }
            }
            load_stage(st[s], jc + kPrefetch);
            __syncthreads();
        }
    }
    if (final_state) {
#pragma unroll
        for (int vb = 0; vb < kNB; ++vb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[sbase + (row0 + i) * kDV + col + kVBlock * vb] = S[vb][i];
    }
}

// Output of every chunk, in parallel: O = Q^ S + O0 with S the chunk's entry
// state, then the gate.  The workgroup copies the chunk's 32 KiB of state
// fragments into LDS once; wave t then forms token rows 16 t .. 16 t + 15 as
// O^T = S^T Q^^T + O0^T (each lane: one token row, 4 consecutive value
// channels) for four value blocks at a time, parks the fp32 tile in LDS, and
// reads it back row-major so that gate loads and output stores are 16 bytes
// per lane and whole 128-byte lines per 8 lanes.  kPair: the workgroup takes
// both chunks of a pair record (8 waves, waves 4..7 on chunk 1 with Q^1' and
// O0_1'), so the pair's entry state is read once.
constexpr int kOutLd = 68;        // fp32 row stride of a wave's 16 x 64 staging tile

template <bool kPair>
__global__ __launch_bounds__(kPair ? 512 : 256) void kda_output_bf16_kernel(
    const bf16 *__restrict__ gate, bf16 *__restrict__ out, const int32_t *__restrict__ cu,
    int N, int T, int H, const uint8_t *__restrict__ ws)
{
    constexpr int kWaves = kPair ? 8 : 4;
    constexpr int kThreads = 64 * kWaves;
    constexpr int kStep = kPair ? kPairTokens : kChunk;
    constexpr size_t kRec = kPair ? kPairRecBytes : kChunkRecBytes;
    __shared__ bf16x8 sb_s[kNumVBlocks * 4][64];
    __shared__ float ot_s[kWaves][kSub][kOutLd];

    // slot-major 1-D grid: workgroup id = slot * H + h.  Workgroups are dealt to
    // the 8 XCDs round-robin, so with H a multiple of 8 every chunk of head h is
    // handled on XCD h % 8, the XCD whose chain workgroups walk head h: the
    // record lines land in the L2 that reads them next
    const int64_t slot = (int64_t)blockIdx.x / H;
    const int h = (int)((int64_t)blockIdx.x % H);
    int n;
    int64_t j;
    if (!slot_to_step<kStep>(cu, N, T, slot, n, j))
        return;
    const SeqInfo si = seq_info(cu, n, T, kStep);
    const int64_t tok0 = si.bos + j * kStep;
    const int64_t lenc = si.len - j * kStep;      // tokens from the slot's start (>= 1)
    const uint8_t *rec = ws + ((int64_t)slot * H + h) * (int64_t)kRec;
    const int tid = threadIdx.x, lane = tid & 63, t = tid >> 6;
    const int m = lane & 15, b = lane >> 4;
    // wave t: chunk c of the slot, its token rows 16 tw .. 16 tw + 15
    const int c = t >> 2, tw = t & 3;
    const uint8_t *qh_rec = rec + (c == 0 ? kOffQH : kOffQH1);
    const uint8_t *o0_rec = rec + (c == 0 ? kOffO0 : kOffO01);

    // state fragments: 2048 x 16 B
    constexpr int kStage = kNumVBlocks * 4 * 64 / kThreads;
    const bf16x8 *sbg = reinterpret_cast<const bf16x8 *>(rec + kOffSB);
    bf16x8 stage[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i)
        stage[i] = sbg[i * kThreads + tid];
    bf16x8 qh[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        qh[ks] = *reinterpret_cast<const bf16x8 *>(qh_rec + (tw * 4 + ks) * kFragBytes +
                                                   lane * 16);
    bf16x4 o0[kNumVBlocks];
#pragma unroll
    for (int blk = 0; blk < kNumVBlocks; ++blk)
        o0[blk] = *reinterpret_cast<const bf16x4 *>(o0_rec + blk * 2048 + (tw >> 1) * 1024 +
                                                    lane * 16 + (tw & 1) * 8);
    // read-back mapping: lane -> row 8 p + lane / 8 of the wave's tile, channels 8 (lane % 8) ..
    // of each 64-channel half; the gate logits of those rows are fetched now,
    // with the other loads (rows past the chunk re-read its last row)
    const int rq = lane >> 3, c8 = 8 * (lane & 7);
    bf16x8 zr[2][2];
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int64_t row = 64 * c + 16 * tw + 8 * p + rq;   // from the slot's first token
            const int64_t rr = row < lenc ? row : lenc - 1;
            zr[half][p] = *reinterpret_cast<const bf16x8 *>(
                gate + ((tok0 + rr) * H + h) * kDV + 64 * half + c8);
        }
    bf16x8 *sbl = &sb_s[0][0];
#pragma unroll
    for (int i = 0; i < kStage; ++i)
        sbl[i * kThreads + tid] = stage[i];
    __syncthreads();

#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
            const int blk = 4 * half + bb;
            f32x4 o = {(float)o0[blk][0], (float)o0[blk][1], (float)o0[blk][2],
                       (float)o0[blk][3]};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                o = mfma16(sb_s[blk * 4 + ks][lane], qh[ks], o);
            *reinterpret_cast<f32x4 *>(&ot_s[t][m][16 * bb + 4 * b]) = o;
        }
        // wave t alone writes and reads back ot_s[t]
        wave_or_group_sync(false);
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int r = 8 * p + rq;
            const int64_t row = 64 * c + 16 * tw + r;
            const f32x4 lo = *reinterpret_cast<const f32x4 *>(&ot_s[t][r][c8]);
            const f32x4 hi = *reinterpret_cast<const f32x4 *>(&ot_s[t][r][c8 + 4]);
            if (row < lenc) {
                const int64_t off = ((tok0 + row) * H + h) * kDV + 64 * half + c8;
                const bf16x8 z = zr[half][p];
                bf16x8 y;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    y[i] = (bf16)(lo[i] * sigmoidf_((float)z[i]));
                    y[4 + i] = (bf16)(hi[i] * sigmoidf_((float)z[4 + i]));
                }
                __builtin_nontemporal_store(y, reinterpret_cast<bf16x8 *>(out + off));
            }
        }
        wave_or_group_sync(false);
    }
}

namespace {

// Persistent prep over every (slot, head) task, a slot being a chunk or a pair
// of chunks (pair): one workgroup per CU (its LDS allows no more), a multiple
// of 8 of them.
template <bool kPro, bool kPair, bool kBwd = false> hipError_t prep_attr()
{
    return hipFuncSetAttribute(
        reinterpret_cast<const void *>(kda_prep_bf16_kernel<kPro, kPair, kBwd>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(PrepSmem));
}

// The persistent prep over n_slots * H tasks on one workgroup per CU (at most
// max_grid workgroups when it is positive, rounded down to a multiple of 8 so
// that task t still runs on XCD t % 8).
// gate, dout, ws_b: per-chunk records (pair = false, pro = 0) that also write
// every chunk's backward record to ws_b (see kda_prep_bf16_kernel); NULL for none.
hipError_t launch_prep(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                       const bf16 *beta, const int32_t *cu, int N, int T, int H, int64_t n_slots,
                       float scale, unsigned pro, uint8_t *ws, hipStream_t stream, bool pair,
                       int max_grid = 0, const bf16 *gate = nullptr, const bf16 *dout = nullptr,
                       uint8_t *ws_b = nullptr)
{
    const hipError_t attr_err = once_per_device<0>([]() -> hipError_t {
        for (hipError_t e : {prep_attr<false, false>(), prep_attr<true, false>(),
                             prep_attr<false, true>(), prep_attr<true, true>(),
                             prep_attr<false, false, true>()})
            if (e != hipSuccess)
                return e;
        return hipSuccess;
    });
    if (attr_err != hipSuccess)
        return attr_err;
    if (n_slots <= 0)
        return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 == hipSuccess)
        e0 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e0 != hipSuccess)
        return e0;
    int64_t prep_grid = cus >= 8 ? cus / 8 * 8 : 8;
    if (max_grid >= 8 && max_grid < prep_grid)
        prep_grid = max_grid / 8 * 8;
    const int64_t n_tasks = n_slots * H;
    const dim3 grid((unsigned)(n_tasks < prep_grid ? n_tasks : prep_grid));
    const size_t lds = sizeof(PrepSmem);
    if (ws_b) {
        if (pro || pair || !gate || !dout)
            return hipErrorInvalidValue;
        hipLaunchKernelGGL((kda_prep_bf16_kernel<false, false, true>), grid, dim3(kPrepThreads),
                           lds, stream, q, k, v, g, beta, cu, N, T, H, n_tasks, scale, 0u, ws, gate,
                           dout, ws_b);
    } else if (pro && pair)
        hipLaunchKernelGGL((kda_prep_bf16_kernel<true, true>), grid, dim3(kPrepThreads), lds,
                           stream, q, k, v, g, beta, cu, N, T, H, n_tasks, scale, pro, ws, nullptr,
                           nullptr, nullptr);
    else if (pro)
        hipLaunchKernelGGL((kda_prep_bf16_kernel<true, false>), grid, dim3(kPrepThreads), lds,
                           stream, q, k, v, g, beta, cu, N, T, H, n_tasks, scale, pro, ws, nullptr,
                           nullptr, nullptr);
    else if (pair)
        hipLaunchKernelGGL((kda_prep_bf16_kernel<false, true>), grid, dim3(kPrepThreads), lds,
                           stream, q, k, v, g, beta, cu, N, T, H, n_tasks, scale, 0u, ws, nullptr,
                           nullptr, nullptr);
    else
        hipLaunchKernelGGL((kda_prep_bf16_kernel<false, false>), grid, dim3(kPrepThreads), lds,
                           stream, q, k, v, g, beta, cu, N, T, H, n_tasks, scale, 0u, ws, nullptr,
                           nullptr, nullptr);
    return hipGetLastError();
}

// The chain over the records in ws, one workgroup per (sequence, head, kNB
// value blocks).  With own_cu each workgroup also reserves LDS it does not
// use, so that no workgroup of a kernel running beside it shares its CU (and
// the CU's memory pipeline, which bounds the chain's step).
constexpr int kChainOwnCuLds = 152 * 1024;   // static + reserved LDS per chain workgroup

// Workgroups of the chain for `units` (sequence, head) units: units rounded up
// to 8 (one per XCD), times the workgroups per unit.
int64_t chain_workgroups(int64_t units, int nb) { return (units + 7) / 8 * 8 * (kNumVBlocks / nb); }

template <int kNB, bool kPair>
hipError_t launch_chain_nb(const float *init, float *final_state, const int32_t *cu, int N,
                           int T, int H, uint8_t *ws, hipStream_t stream, bool own_cu,
                           ChainJob2 job2 = ChainJob2{})
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0)
        return hipSuccess;
    size_t dyn = 0;
    if (own_cu) {
        // the reserved (dynamic) part: kChainOwnCuLds less the kernel's static
        // LDS, allowed once per device
        static std::once_flag attr_once[kMaxDevices];
        static hipError_t attr_err[kMaxDevices];
        static size_t reserve[kMaxDevices];
        int dev = 0;
        hipError_t e = hipGetDevice(&dev);
        if (e != hipSuccess)
            return e;
        if (dev < 0 || dev >= kMaxDevices)
            return hipErrorInvalidDevice;
        std::call_once(attr_once[dev], [dev] {
            const void *fn =
                reinterpret_cast<const void *>(kda_chain_bf16_kernel<false, kNB, kPair>);
            hipFuncAttributes fa{};
            attr_err[dev] = hipFuncGetAttributes(&fa, fn);
            if (attr_err[dev] == hipSuccess && fa.sharedSizeBytes < (size_t)kChainOwnCuLds) {
                reserve[dev] = kChainOwnCuLds - fa.sharedSizeBytes;
                attr_err[dev] = hipFuncSetAttribute(
                    fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)reserve[dev]);
            }
        });
        if (attr_err[dev] != hipSuccess)
            return attr_err[dev];
        dyn = reserve[dev];
    }
    const int64_t wgs = chain_workgroups(units, kNB);
    job2.wgs = (int)wgs;
    hipLaunchKernelGGL((kda_chain_bf16_kernel<false, kNB, kPair>),
                       dim3((unsigned)(job2.ws ? 2 * wgs : wgs)), dim3(chain_threads<kNB>()), dyn,
                       stream, init, final_state, nullptr, 1, cu, T, H, (int)units, ws, job2);
    return hipGetLastError();
}

template <bool kPair>
hipError_t launch_chain_t(const float *init, float *final_state, float *snaps, int snap_interval,
                          const int32_t *cu, int N, int T, int H, uint8_t *ws,
                          hipStream_t stream, bool own_cu)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0)
        return hipSuccess;
    constexpr int kStep = kPair ? kPairTokens : kChunk;
    if (snaps) {
        hipLaunchKernelGGL((kda_chain_bf16_kernel<true, 1, kPair>),
                           dim3((unsigned)chain_workgroups(units, 1)), dim3(chain_threads<1>()),
                           0, stream, init, final_state, snaps, snap_interval / kStep, cu, T, H,
                           (int)units, ws, ChainJob2{});
        return hipGetLastError();
    }
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    if (!own_cu && chain_workgroups(units, 4) >= cus)
        return launch_chain_nb<4, kPair>(init, final_state, cu, N, T, H, ws, stream, false);
    if (!own_cu && chain_workgroups(units, 2) >= cus)
        return launch_chain_nb<2, kPair>(init, final_state, cu, N, T, H, ws, stream, false);
    return launch_chain_nb<1, kPair>(init, final_state, cu, N, T, H, ws, stream, own_cu);
}

// The chain over all units (pair: over pair records; snapshots then at
// multiples of kPairTokens).  When its one-block workgroups outnumber the CUs
// the chain is bound by the operand stream through the device, not by its
// serial depth, and workgroups of 4 (or 2) value blocks stream L once for all
// of them, as long as they still fill the device.
hipError_t launch_chain(const float *init, float *final_state, float *snaps, int snap_interval,
                        const int32_t *cu, int N, int T, int H, uint8_t *ws, hipStream_t stream,
                        bool pair, bool own_cu = false)
{
    return pair ? launch_chain_t<true>(init, final_state, snaps, snap_interval, cu, N, T, H, ws,
                                       stream, own_cu)
                : launch_chain_t<false>(init, final_state, snaps, snap_interval, cu, N, T, H, ws,
                                        stream, own_cu);
}

// The chain of one sequence (T tokens, H heads) on workgroups of 4 value
// blocks that keep their CUs to themselves, for the pipelined long schedule.
hipError_t launch_chain_own4(const float *init, float *final_state, int T, int H, uint8_t *ws,
                             hipStream_t stream, bool pair)
{
    return pair ? launch_chain_nb<4, true>(init, final_state, nullptr, 1, T, H, ws, stream, true)
                : launch_chain_nb<4, false>(init, final_state, nullptr, 1, T, H, ws, stream, true);
}

// Two chains over per-chunk records of the same sequences in one launch: over
// ws_a from init_a (no final state) and over ws_b from init_b, its final state
// to final_b.  The workgroups per unit follow the rule above for the
// launch's two chains together.
hipError_t launch_chain_two(const float *init_a, uint8_t *ws_a, const float *init_b,
                            float *final_b, uint8_t *ws_b, const int32_t *cu, int N, int T, int H,
                            hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    if (units <= 0)
        return hipSuccess;
    int dev = 0, cus = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    const ChainJob2 job2{init_b, final_b, ws_b, 0};
    if (2 * chain_workgroups(units, 4) >= cus)
        return launch_chain_nb<4, false>(init_a, nullptr, cu, N, T, H, ws_a, stream, false, job2);
    if (2 * chain_workgroups(units, 2) >= cus)
        return launch_chain_nb<2, false>(init_a, nullptr, cu, N, T, H, ws_a, stream, false, job2);
    return launch_chain_nb<1, false>(init_a, nullptr, cu, N, T, H, ws_a, stream, false, job2);
}

hipError_t launch_output(const bf16 *gate, bf16 *out, const int32_t *cu, int N, int T, int H,
                         int64_t n_slots, const uint8_t *ws, hipStream_t stream, bool pair)
{
    if (n_slots <= 0 || H <= 0)
        return hipSuccess;
    if (pair)
        hipLaunchKernelGGL(kda_output_bf16_kernel<true>, dim3((unsigned)(n_slots * H)),
                           dim3(512), 0, stream, gate, out, cu, N, T, H, ws);
    else
        hipLaunchKernelGGL(kda_output_bf16_kernel<false>, dim3((unsigned)(n_slots * H)),
                           dim3(256), 0, stream, gate, out, cu, N, T, H, ws);
    return hipGetLastError();
}

// ---- long single sequences: output beside the chain ---------------------------
//
// On one long sequence the chain walks thousands of chunks on H * 8
// workgroups while the rest of the device idles.  The chain then runs on a
// second stream in segments of at least kSegTokens tokens, each starting from the
// previous segment's final state (fp32, written to final_state and read back
// unchanged, so the result is bitwise that of one chain), and the caller's
// stream runs the output kernel of each segment as soon as that segment's
// chain is done, beside the chain of the next.  Records, inputs and outputs
// of a segment are addressed by offsetting the base pointers, so the kernels
// see an ordinary one-sequence call.
//
// The second stream and a pool of events are created once per device, at the
// first such call, and kept until the process ends; a mutex orders the
// record / wait / launch sequences of concurrent host threads.
constexpr int64_t kSegTokens = 512 * kChunk;
constexpr int64_t kMinSegmentedTokens = 2 * kSegTokens;
constexpr int kMaxSegments = 32;
// segments of the pipelined schedule: fewer and longer than the chain's alone,
// since each also ends a prep launch, but not so few that the last segment's
// chain and output, which run after all prep, take long (measured on 1M tokens
// x 16 heads, ms per call: 6 segments 19.0, 9 18.5-18.8, 11 18.4-18.6, 16
// 18.2-18.5, 31 18.5-18.9, 59 19.2-19.7)
constexpr int kPipeSegments = 16;

struct AuxStream {
    bool ready = false;
    hipStream_t stream = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    hipEvent_t seg[kMaxSegments] = {};    // a segment's chain is done (second stream)
    hipEvent_t pseg[kMaxSegments] = {};   // a segment's prep is done (caller's stream)
};
std::mutex g_aux_mutex;
AuxStream g_aux[kMaxDevices];

hipError_t aux_stream(AuxStream *&out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    AuxStream &a = g_aux[dev];
    if (!a.ready) {
        e = hipStreamCreateWithFlags(&a.stream, hipStreamNonBlocking);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&a.fork, hipEventDisableTiming);
        if (e == hipSuccess)
            e = hipEventCreateWithFlags(&a.join, hipEventDisableTiming);
        for (int i = 0; i < kMaxSegments && e == hipSuccess; ++i) {
            e = hipEventCreateWithFlags(&a.seg[i], hipEventDisableTiming);
            if (e == hipSuccess)
                e = hipEventCreateWithFlags(&a.pseg[i], hipEventDisableTiming);
        }
        if (e != hipSuccess) {
            // release what was created, so that a later call starts afresh
            for (hipEvent_t *set : {a.seg, a.pseg})
                for (int i = 0; i < kMaxSegments; ++i)
                    if (set[i]) {
                        (void)hipEventDestroy(set[i]);
                        set[i] = nullptr;
                    }
            for (hipEvent_t *ev : {&a.fork, &a.join})
                if (*ev) {
                    (void)hipEventDestroy(*ev);
                    *ev = nullptr;
                }
            if (a.stream) {
                (void)hipStreamDestroy(a.stream);
                a.stream = nullptr;
            }
            return e;
        }
        a.ready = true;
    }
    out = &a;
    return hipSuccess;
}

// True when `stream` is recording a graph capture (or when that cannot be
// told, so that the single-stream schedule, correct everywhere, is taken).
bool stream_capturing(hipStream_t stream)
{
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cs) != hipSuccess) {
        (void)hipGetLastError();
        return true;
    }
    return cs != hipStreamCaptureStatusNone;
}

}  // namespace

hipError_t launch_chunk_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                             const bf16 *beta, const bf16 *gate, const float *init, bf16 *out,
                             float *final_state, float *snaps, int snap_interval,
                             const int32_t *cu, int N, int T, int H, int64_t n_slots,
                             float scale, unsigned pro, void *workspace, hipStream_t stream,
                             bool pair, bool allow_aux)
{
    uint8_t *ws = static_cast<uint8_t *>(workspace);
    const int64_t step = pair ? kPairTokens : kChunk;                 // tokens per slot
    const int64_t rec_bytes = pair ? (int64_t)kPairRecBytes : (int64_t)kChunkRecBytes;
    // segments need one sequence without cu_seqlens, no snapshots and a final
    // state buffer to hand the state over in; a stream that is being captured
    // into a graph keeps the single-stream schedule, so that no work of the
    // shared auxiliary stream is pulled into the capture
    const bool segmented = allow_aux && !cu && N == 1 && !snaps && final_state &&
                           n_slots * step >= kMinSegmentedTokens && !stream_capturing(stream);
    hipError_t e = hipSuccess;
    if (!segmented) {
        e = launch_prep(q, k, v, g, beta, cu, N, T, H, n_slots, scale, pro, ws, stream, pair);
        if (e == hipSuccess)
            e = launch_chain(init, final_state, snaps, snap_interval, cu, N, T, H, ws, stream,
                             pair);
        if (e == hipSuccess)
            e = launch_output(gate, out, cu, N, T, H, n_slots, ws, stream, pair);
        return e;
    }
    int dev = 0, cus = 0;
    e = hipGetDevice(&dev);
    if (e == hipSuccess)
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess)
        return e;
    // Pipelined when the chain's 4-block workgroups (one CU each) need at most a
    // quarter of the device: prep runs segment by segment on the other CUs, and
    // each segment's chain follows its prep on the second stream while prep
    // goes on with the next segment.  A segment then holds whole rounds of prep
    // tasks (a multiple of prep_grid / gcd(prep_grid, H) slots).
    const int64_t chain_cus = chain_workgroups(H, 4);
    const bool pipelined = chain_cus * 4 <= cus;
    const int prep_grid = pipelined ? (int)((cus - chain_cus) / 8 * 8) : 0;
    int64_t seg = (n_slots + kMaxSegments - 1) / kMaxSegments;       // slots per segment
    seg = seg * step < kSegTokens ? kSegTokens / step : seg;
    if (pipelined) {
        const int64_t quantum = prep_grid / std::gcd((int64_t)prep_grid, (int64_t)H);
        seg = (n_slots + kPipeSegments - 1) / kPipeSegments;
        seg = seg * step < kSegTokens ? kSegTokens / step : seg;
        seg = (seg + quantum - 1) / quantum * quantum;
    }
    const int64_t nseg = (n_slots + seg - 1) / seg;                   // at most kMaxSegments
    struct Seg {
        int64_t slot0, ns, tok0;
        int Ts;
        uint8_t *ws;
    };
    auto seg_at = [&](int64_t s) {
        Seg r;
        r.slot0 = s * seg;
        r.ns = n_slots - r.slot0 < seg ? n_slots - r.slot0 : seg;
        r.tok0 = r.slot0 * step;
        r.Ts = (int)(T - r.tok0 < r.ns * step ? T - r.tok0 : r.ns * step);
        r.ws = ws + r.slot0 * H * rec_bytes;
        return r;
    };
    std::lock_guard<std::mutex> lock(g_aux_mutex);
    AuxStream *aux = nullptr;
    e = aux_stream(aux);
    if (e != hipSuccess)
        return e;
    if (pipelined) {
        // caller's stream: prep 0, prep 1, output 0, prep 2, output 1, ...; second
        // stream: chain s once prep s is done.  Output s - 1 waits for chain s - 1,
        // which ran beside prep s.
        for (int64_t s = 0; s <= nseg && e == hipSuccess; ++s) {
            if (s < nseg) {
                const Seg c = seg_at(s);
                const int64_t t0 = c.tok0 * H;
                e = launch_prep(q + t0 * kDK, k + t0 * kDK, v + t0 * kDV, g + t0 * kDK, beta + t0,
                                nullptr, 1, c.Ts, H, c.ns, scale, pro, c.ws, stream, pair,
                                prep_grid);
                if (e == hipSuccess)
                    e = hipEventRecord(aux->pseg[s], stream);
                if (e == hipSuccess)
                    e = hipStreamWaitEvent(aux->stream, aux->pseg[s], 0);
                if (e == hipSuccess) {
                    // the last segment's chain has no prep beside it, only the
                    // outputs of the segment before, and bounds the end of the
                    // call: workgroups of 2 value blocks (twice the CUs, each
                    // still to itself) walk it faster than those of 4
                    if (s + 1 == nseg)
                        e = (pair ? launch_chain_nb<2, true>
                                  : launch_chain_nb<2, false>)(
                            s == 0 ? init : final_state, final_state, nullptr, 1, c.Ts, H, c.ws,
                            aux->stream, true, ChainJob2{});
                    else
                        e = launch_chain_own4(s == 0 ? init : final_state, final_state, c.Ts, H,
                                              c.ws, aux->stream, pair);
                }
                if (e == hipSuccess)
                    e = hipEventRecord(aux->seg[s], aux->stream);
            }
            if (s >= 1 && e == hipSuccess) {
                const Seg c = seg_at(s - 1);
                e = hipStreamWaitEvent(stream, aux->seg[s - 1], 0);
                if (e == hipSuccess)
                    e = launch_output(gate + c.tok0 * H * kDV, out + c.tok0 * H * kDV, nullptr, 1,
                                      c.Ts, H, c.ns, c.ws, stream, pair);
            }
        }
    } else {
        e = launch_prep(q, k, v, g, beta, cu, N, T, H, n_slots, scale, pro, ws, stream, pair);
        if (e == hipSuccess)
            e = hipEventRecord(aux->fork, stream);
        if (e == hipSuccess)
            e = hipStreamWaitEvent(aux->stream, aux->fork, 0);
        for (int64_t s = 0; s < nseg && e == hipSuccess; ++s) {
            const Seg c = seg_at(s);
            e = launch_chain(s == 0 ? init : final_state, final_state, nullptr, 0, nullptr, 1,
                             c.Ts, H, c.ws, aux->stream, pair, true);
            if (e == hipSuccess)
                e = hipEventRecord(aux->seg[s], aux->stream);
            if (e == hipSuccess)
                e = hipStreamWaitEvent(stream, aux->seg[s], 0);
            if (e == hipSuccess)
                e = launch_output(gate + c.tok0 * H * kDV, out + c.tok0 * H * kDV, nullptr, 1,
                                  c.Ts, H, c.ns, c.ws, stream, pair);
        }
    }
    if (e != hipSuccess) {
        // after a failure part way, still order the caller's stream after
        // whatever reached the second stream, which reads the workspace
        if (hipEventRecord(aux->join, aux->stream) == hipSuccess)
            (void)hipStreamWaitEvent(stream, aux->join, 0);
    }
    return e;
}

// Backward: forward records (prep + chain give every chunk's entry state, or
// the caller passes those of its kda_chunk_fwd call), backward records in
// reverse chunk order (-L^T, Q^^T dO, dec), the same chain over them from
// dS_final (the state gradient on exit of every chunk, and dS_0), then the
// per-chunk gradients.
hipError_t launch_chunk_bwd_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                                 const bf16 *beta, const bf16 *gate, const float *init,
                                 const bf16 *dout, const float *dfinal, bf16 *dq, bf16 *dk,
                                 bf16 *dv, bf16 *dg, bf16 *dbeta, bf16 *dgate, float *dinit,
                                 const int32_t *cu, int N, int T, int H, int64_t n_slots,
                                 float scale, void *fwd_records, void *workspace,
                                 hipStream_t stream)
{
    const size_t rec_bytes = (size_t)n_slots * (size_t)H * kChunkRecBytes;
    uint8_t *ws_f = fwd_records ? static_cast<uint8_t *>(fwd_records)
                                : static_cast<uint8_t *>(workspace);
    uint8_t *ws_b = fwd_records ? static_cast<uint8_t *>(workspace)
                                : static_cast<uint8_t *>(workspace) + rec_bytes;
    hipError_t e = hipSuccess;
    if (fwd_records) {
        e = launch_bwd_prep_bf16(gate, dout, cu, N, T, H, n_slots, ws_f, ws_b, stream);
        if (e == hipSuccess)
            e = launch_chain(dfinal, dinit, nullptr, 0, cu, N, T, H, ws_b, stream, false);
    } else {
        // The state-gradient recurrence needs the forward records but not the
        // forward states, and the chain writes only SB: the prep writes the
        // backward records too, and then one launch runs the forward chain
        // (every chunk's entry state) and the backward chain side by side.
        e = launch_prep(q, k, v, g, beta, cu, N, T, H, n_slots, scale, 0u, ws_f, stream, false, 0,
                        gate, dout, ws_b);
        if (e == hipSuccess)
            e = launch_chain_two(init, ws_f, dfinal, dinit, ws_b, cu, N, T, H, stream);
    }
    if (e == hipSuccess)
        e = launch_grad_bf16(q, k, v, g, beta, gate, dout, dq, dk, dv, dg, dbeta, dgate, cu, N,
                             T, H, n_slots, scale, ws_f, ws_b, stream);
    return e;
}

}  // namespace kda
