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
// Two kernels:
//   prep  (512 threads per (chunk slot, head); all chunks in parallel):
//         G, A and P (bf16 MFMA), T (fp32 substitution), W and U~ (MFMA), then
//         L, Bm, Q^ and O0 (MFMA) written as the chain's operands.
//   chain (256 threads per (sequence, head, 16-wide value block)): walks the
//         chunks in order.  Wave w keeps rows 32 w .. 32 w + 31 of the fp32
//         state slice in its accumulators and computes those rows of
//         S' = dec S + Bm - L S and rows 16 w .. 16 w + 15 of O = Q^ S + O0;
//         the four waves exchange the new state as bf16 MFMA fragments
//         through 8 KiB of LDS, one barrier per chunk.  The operands of the
//         next chunks are prefetched into registers.
#include "kda_internal.h"

#include <mutex>

namespace kda {

namespace {

constexpr int kPrepThreads = 512;
constexpr int kRowLd = 136;   // bf16 row stride of row-major 64 x 128 tiles
constexpr int kColLd = 72;    // bf16 row stride of channel-major 128 x 64 tiles
constexpr int kALd = 65;      // fp32 row stride of A and T

struct PrepSmem {
    // -- live in phases 1-2 only; T and its scratch reuse this space afterwards
    bf16 KR[kChunk][kRowLd];      // k e^{G - B_i(r)}      (row operand of A)
    bf16 KCD[kChunk][kRowLd];     // k e^{B_i(r) - G}      (column operand, diagonal ref.)
    float F[6][kDK];              // e^{B_i - B_j}, i > j  (pairs 10 20 21 30 31 32)
    // -- live until the end
    bf16 QR[kChunk][kRowLd];      // q e^{G - B_i(r)}      (row operand of P; Q e^G later)
    bf16 XB[kDK][kColLd];         // beta k e^G, channel-major
    bf16 VB[kDV][kColLd];         // beta v, channel-major
    bf16 KPT[kDK][kColLd];        // K' = k e^{G_end - G}, channel-major
    bf16 PM[kChunk][kColLd];      // scale P, lower incl., zero above
    float AM[kChunk][kALd];       // diag(beta) A, strict lower (scan scratch in phase 1)
    float Bref[4][kDK];           // B_0 = 0, B_1..B_3
    float Gend[kDK];
    float beta[kChunk];
};

struct TSmem {                    // overlays KR / KCD / F after phase 2
    float TM[kChunk][kALd];
    float X[3][kSub][kSub + 1];
};
static_assert(sizeof(TSmem) <= 2 * sizeof(bf16) * kChunk * kRowLd + 6 * kDK * sizeof(float),
              "T overlay fits");

__device__ __forceinline__ int pair_index(int i, int j) { return (i * (i - 1)) / 2 + j; }

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

__device__ __forceinline__ bf16x4 to_bf16x4(const f32x4 &a, float s)
{
    return bf16x4{(bf16)(s * a[0]), (bf16)(s * a[1]), (bf16)(s * a[2]), (bf16)(s * a[3])};
}

// Chunk slot -> (sequence, chunk index).  Returns false for an unused slot.
__device__ __forceinline__ bool slot_to_chunk(const int32_t *cu, int N, int T, int64_t slot,
                                              int &n, int64_t &j)
{
    if (cu) {
        int lo = 0, hi = N - 1;
        while (lo < hi) {                       // largest n with cu[n]/C + n <= slot
            const int mid = (lo + hi + 1) >> 1;
            if ((int64_t)cu[mid] / kChunk + mid <= slot)
                lo = mid;
            else
                hi = mid - 1;
        }
        n = lo;
        j = slot - ((int64_t)cu[n] / kChunk + n);
        return (int64_t)cu[n + 1] - cu[n] > j * kChunk;
    }
    const int64_t nck = (T + kChunk - 1) / kChunk;
    n = (int)(slot / nck);
    j = slot % nck;
    return n < N;
}

}  // namespace

__global__ __launch_bounds__(kPrepThreads) void kda_prep_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, const int32_t *__restrict__ cu,
    int N, int T, int H, float scale, uint8_t *__restrict__ ws)
{
    extern __shared__ __align__(16) uint8_t smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);
    TSmem &ts = *reinterpret_cast<TSmem *>(smem_raw);

    const int64_t slot = blockIdx.x;
    const int h = blockIdx.y;
    int n;
    int64_t j;
    if (!slot_to_chunk(cu, N, T, slot, n, j))
        return;
    const SeqInfo si = seq_info(cu, n, T, kChunk);
    const int64_t tok0 = si.bos + j * kChunk;
    const int len = (int)((si.len - j * kChunk) < kChunk ? (si.len - j * kChunk) : kChunk);
    uint8_t *rec = ws + ((int64_t)slot * H + h) * (int64_t)kRecBytes;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int m = lane & 15, b = lane >> 4;
    const int64_t tstride = (int64_t)H * kDK;   // elements between consecutive tokens

    // ---- phase 1: loads, cumulative log-decay, elementwise operands -----------
    // thread -> channels 8 cg .. 8 cg + 7 of rows 2 rg, 2 rg + 1
    const int cg = tid & 15, rg = tid >> 4;
    float qv[2][8], kv[2][8], vv[2][8], Gl[2][8];
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
        const int r = 2 * rg + rr;
        bf16x8 q8 = {}, k8 = {}, v8 = {}, g8 = {};
        if (r < len) {
            const int64_t o = (tok0 + r) * tstride + (int64_t)h * kDK + 8 * cg;
            q8 = *reinterpret_cast<const bf16x8 *>(q + o);
            k8 = *reinterpret_cast<const bf16x8 *>(k + o);
            v8 = *reinterpret_cast<const bf16x8 *>(v + o);
            g8 = *reinterpret_cast<const bf16x8 *>(g + o);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qv[rr][e] = (float)q8[e];
            kv[rr][e] = (float)k8[e];
            vv[rr][e] = (float)v8[e];
            Gl[rr][e] = (float)g8[e] + (rr ? Gl[0][e] : 0.f);
        }
    }
    if (tid < kChunk)
        sm.beta[tid] = tid < len ? (float)beta[(tok0 + tid) * H + h] : 0.f;
    {
        // zero P (the upper blocks stay zero) while the loads land
        bf16 *pm = &sm.PM[0][0];
        for (int i = tid; i < kChunk * kColLd; i += kPrepThreads)
            pm[i] = (bf16)0.f;
    }
    float(*tot)[kDK] = reinterpret_cast<float(*)[kDK]>(&sm.AM[0][0]);   // [32][128]
    *reinterpret_cast<f32x4 *>(&tot[rg][8 * cg]) = f32x4{Gl[1][0], Gl[1][1], Gl[1][2], Gl[1][3]};
    *reinterpret_cast<f32x4 *>(&tot[rg][8 * cg + 4]) = f32x4{Gl[1][4], Gl[1][5], Gl[1][6], Gl[1][7]};
    __syncthreads();
    if (tid < kDK) {
        // exclusive scan over the 32 row pairs of channel tid
        float t[32];
#pragma unroll
        for (int x = 0; x < 32; ++x)
            t[x] = tot[x][tid];
        float run = 0.f;
#pragma unroll
        for (int x = 0; x < 32; ++x) {
            const float nx = run + t[x];
            tot[x][tid] = run;
            if (x == 8)
                sm.Bref[1][tid] = run;
            if (x == 16)
                sm.Bref[2][tid] = run;
            if (x == 24)
                sm.Bref[3][tid] = run;
            run = nx;
        }
        sm.Bref[0][tid] = 0.f;
        sm.Gend[tid] = run;
    }
    __syncthreads();
    {
        const int bi = rg >> 3;                      // subtile of both rows
        float ex[8], Bi[8], eB[8], eGB[8];
        const f32x4 e0 = *reinterpret_cast<const f32x4 *>(&tot[rg][8 * cg]);
        const f32x4 e1 = *reinterpret_cast<const f32x4 *>(&tot[rg][8 * cg + 4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            ex[e] = e0[e];
            ex[4 + e] = e1[e];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            Bi[e] = sm.Bref[bi][8 * cg + e];
            eB[e] = __expf(Bi[e]);                                   // e^{B_i} <= 1
            eGB[e] = __expf(sm.Gend[8 * cg + e] - Bi[e]);             // e^{G_end - B_i} <= 1
        }
        bf16 xb[2][8], vb[2][8], kp[2][8];
#pragma unroll
        for (int rr = 0; rr < 2; ++rr) {
            const int r = 2 * rg + rr;
            const float br = sm.beta[r];
            bf16x8 kr8, qr8, kc8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float G = ex[e] + Gl[rr][e];
                const float fr = __expf(G - Bi[e]);          // e^{G - B_i} in [e^-80, 1]
                const float fc = __frcp_rn(fr);              // e^{B_i - G} in [1, e^80]
                kr8[e] = (bf16)(kv[rr][e] * fr);
                qr8[e] = (bf16)(qv[rr][e] * fr);
                kc8[e] = (bf16)(kv[rr][e] * fc);
                xb[rr][e] = (bf16)(br * kv[rr][e] * (fr * eB[e]));         // beta k e^G
                vb[rr][e] = (bf16)(br * vv[rr][e]);
                kp[rr][e] = (bf16)(kv[rr][e] * (eGB[e] * fc));             // k e^{G_end - G}
            }
            *reinterpret_cast<bf16x8 *>(&sm.KR[r][8 * cg]) = kr8;
            *reinterpret_cast<bf16x8 *>(&sm.QR[r][8 * cg]) = qr8;
            *reinterpret_cast<bf16x8 *>(&sm.KCD[r][8 * cg]) = kc8;
        }
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int c = 8 * cg + e;
            *reinterpret_cast<bf16x2 *>(&sm.XB[c][2 * rg]) = bf16x2{xb[0][e], xb[1][e]};
            *reinterpret_cast<bf16x2 *>(&sm.VB[c][2 * rg]) = bf16x2{vb[0][e], vb[1][e]};
            *reinterpret_cast<bf16x2 *>(&sm.KPT[c][2 * rg]) = bf16x2{kp[0][e], kp[1][e]};
        }
    }
    if (tid < kDK) {
        int p = 0;
#pragma unroll
        for (int i = 1; i < 4; ++i)
#pragma unroll
            for (int jj = 0; jj < i; ++jj)
                sm.F[p++][tid] = __expf(sm.Bref[i][tid] - sm.Bref[jj][tid]);
    }
    __syncthreads();

    // ---- phase 2: 16 x 16 blocks of A and P (bf16 MFMA, fp32 accumulate) -------
    for (int blk = wave; blk < 10; blk += kPrepThreads / 64) {
        // blk -> (i, jb): 0:(0,0) 1:(1,0) 2:(1,1) 3:(2,0) 4:(2,1) 5:(2,2) 6:(3,0) ...
        const int i = blk < 1 ? 0 : blk < 3 ? 1 : blk < 6 ? 2 : 3;
        const int jb = blk - (i * (i + 1)) / 2;
        f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 32 * ks + 8 * b;
            const bf16x8 ar = lds8(&sm.KR[16 * i + m][ch]);
            const bf16x8 aq = lds8(&sm.QR[16 * i + m][ch]);
            bf16x8 bc = lds8(&sm.KCD[16 * jb + m][ch]);
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
            sm.AM[row][col] = (jb < i || col < row) ? sm.beta[row] * accA[e] : 0.f;
            sm.PM[row][col] = (bf16)((jb < i || col <= row) ? scale * accP[e] : 0.f);
        }
    }
    __syncthreads();

    // ---- phase 3: T = (I + A)^-1 ------------------------------------------------
    if (wave == 0) {
        // diagonal 16 x 16 blocks by forward substitution, one column per lane;
        // x[s] = 0 for s < col, so the full-range sums only add zeros there
        const int blk = lane >> 4, col = lane & 15, o = 16 * blk;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s)
                acc -= sm.AM[o + r][o + s] * x[s];
            x[r] = (r < col) ? 0.f : acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            ts.TM[o + r][o + col] = x[r];
    } else if (wave <= 2) {
        // T_01 and T_23 are read by the W / U~ products: zero them
        const int t = tid - 64, o = (wave == 1) ? 0 : 32;
        for (int e = t % 64; e < 256; e += 64)
            ts.TM[o + e / 16][o + 16 + e % 16] = 0.f;
    }
    __syncthreads();
    {
        // off-diagonal blocks by distance: T_ab = -T_aa (sum_{mm=b}^{a-1} A_a,mm T_mm,b)
        const int rr = (tid >> 4) & 15, cc = tid & 15, grp = tid >> 8;
        for (int dist = 1; dist < 4; ++dist) {
            const int nb = 4 - dist;
            for (int p = grp; p < nb; p += 2) {
                const int a = p + dist, bb = p;
                float acc = 0.f;
                for (int mm = bb; mm < a; ++mm)
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        acc += sm.AM[16 * a + rr][16 * mm + s] * ts.TM[16 * mm + s][16 * bb + cc];
                ts.X[p][rr][cc] = acc;
            }
            __syncthreads();
            for (int p = grp; p < nb; p += 2) {
                const int a = p + dist, bb = p;
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc -= ts.TM[16 * a + rr][16 * a + s] * ts.X[p][s][cc];
                ts.TM[16 * a + rr][16 * bb + cc] = acc;
            }
            __syncthreads();
        }
    }

    // ---- phase 4: W = T X and U~ = T V for the wave's 16 channels --------------
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
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] = (bf16)ts.TM[16 * mt + m][32 * ks + 8 * b + e];
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
        // L^T rows 16 nt.. = W^T K'  ->  -L fragments (mt, kq), elements 4 half .. 4 half + 3
        // Bm columns 16 nt.. = K'^T U~ ->  Bm of value block nt
#pragma unroll
        for (int mt = 0; mt < 8; ++mt) {
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
            *reinterpret_cast<bf16x4 *>(rec + kOffLN + (mt * 4 + kq) * kFragBytes + lane * 16 +
                                        half * 8) = to_bf16x4(l, -1.f);
            *reinterpret_cast<bf16x4 *>(rec + kOffBM + nt * 4096 + (mt >> 1) * 1024 + lane * 16 +
                                        (mt & 1) * 8) = to_bf16x4(bm, 1.f);
        }
        // Q^ = scale Q e^G - P W  (as Q^^T rows 16 nt..)  and  O0 = P U~ for value block nt
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            bf16x8 pf[2];
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                pf[ks] = perm8(&sm.PM[16 * mt + m][0], ks, b);
            // scale Q e^G at row 16 mt + m, channels 16 nt + 4 b .. + 3, from q e^{G - B_mt}
            const bf16x4 qr = *reinterpret_cast<const bf16x4 *>(&sm.QR[16 * mt + m][16 * nt + 4 * b]);
            f32x4 qh;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                qh[i] = -scale * (float)qr[i] * __expf(sm.Bref[mt][16 * nt + 4 * b + i]);
            f32x4 o0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                qh = mfma16(wf[ks], pf[ks], qh);   // (P W)^T - (scale Q e^G)^T
                o0 = mfma16(uf[ks], pf[ks], o0);   // (P U~)^T
            }
            *reinterpret_cast<bf16x4 *>(rec + kOffQH + (mt * 4 + kq) * kFragBytes + lane * 16 +
                                        half * 8) = to_bf16x4(qh, -1.f);
            *reinterpret_cast<bf16x4 *>(rec + kOffO0 + nt * 2048 + mt * 512 + lane * 8) =
                to_bf16x4(o0, 1.f);
        }
    }
    if (tid < kDK)
        reinterpret_cast<float *>(rec + kOffDEC)[tid] = __expf(sm.Gend[tid]);
}

namespace {

// Chain workgroup: 4 compute waves and 1 store wave.  Compute wave w keeps
// state rows 32 w .. 32 w + 31 (two 16-row tiles) and produces output token
// rows 16 w .. 16 w + 15 of each chunk; it only ever loads from global memory,
// and writes its gated outputs to LDS.  The store wave copies each chunk's
// outputs from LDS to global memory one chunk later.  Keeping loads and stores
// in different waves lets the compiler wait for exactly the prefetched stage
// it needs (with both kinds pending it can only wait for everything).
constexpr int kComputeWaves = 4;
constexpr int kChainThreads = 64 * (kComputeWaves + 1);
constexpr int kPrefetch = 3;         // chunks of operands in flight per compute wave

struct ChainStage {
    bf16x8 ln[2][4];   // -L rows of the wave's two state tiles, 4 dk k-steps each
    bf16x8 qh[4];      // Q^ rows of the wave's output tile
    bf16x8 bm;         // Bm of the wave's 32 state rows, this value block
    f32x4 dec[2];      // e^{G_end} of the wave's state rows
    bf16x4 o0;         // O0 of the wave's output token row, 4 value channels
    bf16x4 z;          // gate logits of the same token row and channels
};

// Every load is unconditional (rows past a partial chunk re-read the chunk's
// last row), so each loop iteration issues the same memory operations.
__device__ __forceinline__ void chain_load(ChainStage &st, const uint8_t *rec, const bf16 *gate,
                                           int64_t tok0, int64_t lenc, int H, int h, int w,
                                           int lane, int blk)
{
    const int m = lane & 15, b = lane >> 4;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            st.ln[t][ks] = *reinterpret_cast<const bf16x8 *>(
                rec + kOffLN + ((2 * w + t) * 4 + ks) * kFragBytes + lane * 16);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        st.qh[ks] = *reinterpret_cast<const bf16x8 *>(rec + kOffQH + (w * 4 + ks) * kFragBytes +
                                                      lane * 16);
    st.bm = *reinterpret_cast<const bf16x8 *>(rec + kOffBM + blk * 4096 + w * 1024 + lane * 16);
#pragma unroll
    for (int t = 0; t < 2; ++t)
        st.dec[t] = *reinterpret_cast<const f32x4 *>(rec + kOffDEC + (32 * w + 16 * t + 4 * b) * 4);
    st.o0 = *reinterpret_cast<const bf16x4 *>(rec + kOffO0 + blk * 2048 + w * 512 + lane * 8);
    const int64_t row = 16 * w + m;
    const int64_t r = row < lenc ? row : lenc - 1;
    st.z = *reinterpret_cast<const bf16x4 *>(gate + ((tok0 + r) * H + h) * kDV + kVBlock * blk +
                                             4 * b);
}

}  // namespace

__global__ __launch_bounds__(kChainThreads) void kda_chain_bf16_kernel(
    const bf16 *__restrict__ gate, const float *__restrict__ init, bf16 *__restrict__ out,
    float *__restrict__ final_state, const int32_t *__restrict__ cu, int T, int H, int units,
    const uint8_t *__restrict__ ws)
{
    __shared__ bf16x8 sbuf[2][4][64];                 // state as 4 k-step fragments
    __shared__ bf16x4 ybuf[2][kChunk][kVBlock / 4];   // gated outputs of one chunk

    // all value blocks of one (sequence, head) land on the same XCD (blocks are
    // dealt to the 8 XCDs round-robin), so they share that XCD's L2
    const int id = blockIdx.x;
    const int xcd = id & 7, qid = id >> 3;
    const int unit = (qid >> 3) * 8 + xcd;
    const int blk = qid & 7;
    if (unit >= units)
        return;
    const int n = unit / H, h = unit % H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int m = lane & 15, b = lane >> 4;
    const SeqInfo si = seq_info(cu, n, T, kChunk);
    const int64_t nch = (si.len + kChunk - 1) / kChunk;

    // the chunk loop runs in rounds of kPrefetch iterations; iterations past the
    // last chunk (at most kPrefetch - 1) leave the state unchanged and store nothing
    const int64_t niter = (nch + kPrefetch - 1) / kPrefetch * kPrefetch;
    if (w == kComputeWaves) {
        // store wave: lane r copies token row r of a finished chunk (32 bytes)
        __syncthreads();
        for (int64_t jc = 0; jc <= niter; ++jc) {
            if (jc > 0 && lane < si.len - (jc - 1) * kChunk) {
                const bf16x8 *src = reinterpret_cast<const bf16x8 *>(&ybuf[(jc - 1) & 1][lane][0]);
                bf16x8 *dst = reinterpret_cast<bf16x8 *>(
                    out + ((si.bos + (jc - 1) * kChunk + lane) * H + h) * kDV + kVBlock * blk);
                dst[0] = src[0];
                dst[1] = src[1];
            }
            if (jc < niter)
                __syncthreads();
        }
        return;
    }

    const int64_t sbase = (int64_t)unit * (kDK * kDV);
    const int col = kVBlock * blk + m;
    // state tile t of this wave: rows 32 w + 16 t + 4 b + i, column col
    f32x4 S[2];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = init ? init[sbase + (32 * w + 16 * t + 4 * b + i) * kDV + col] : 0.f;
    sbuf[0][w][lane] = acc_to_frag(S[0], S[1]);
    __syncthreads();

    // the scheduling barriers keep each stage's loads together and in stage
    // order, in the prologue and in the loop alike, so the loop-entry wait
    // state is the same on both paths and every wait stays partial
    auto load_stage = [&](ChainStage &stage, int64_t jc) {
        const int64_t jl = jc < nch ? jc : nch - 1;
        __builtin_amdgcn_sched_barrier(0);
        chain_load(stage, ws + ((si.slot0 + jl) * H + h) * (int64_t)kRecBytes, gate,
                   si.bos + jl * kChunk, si.len - jl * kChunk, H, h, w, lane, blk);
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
            const bool live = jc < nch;
            const ChainStage &c = st[s];
            const bf16x8 *sb = &sbuf[jc & 1][0][lane];
            // S' = dec S + Bm - L S for the wave's 32 rows
            f32x4 acc[2];
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    acc[t][i] = c.dec[t][i] * S[t][i] + (float)c.bm[4 * t + i];
            // O^T = S^T Q^^T + O0^T: this lane gets token row 16 w + m, value
            // channels 16 blk + 4 b .. + 3 (the state fragments serve as A)
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                o[i] = (float)c.o0[i];
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const bf16x8 f = sb[ks * 64];
                acc[0] = mfma16(c.ln[0][ks], f, acc[0]);
                acc[1] = mfma16(c.ln[1][ks], f, acc[1]);
                o = mfma16(f, c.qh[ks], o);
            }
            if (live) {
                S[0] = acc[0];
                S[1] = acc[1];
            }
            sbuf[(jc + 1) & 1][w][lane] = acc_to_frag(S[0], S[1]);
            bf16x4 y;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                y[i] = (bf16)(o[i] * __builtin_amdgcn_rcpf(1.0f + __expf(-(float)c.z[i])));
            ybuf[jc & 1][16 * w + m][b] = y;
            load_stage(st[s], jc + kPrefetch);
            __syncthreads();
        }
    }
    if (final_state) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[sbase + (32 * w + 16 * t + 4 * b + i) * kDV + col] = S[t][i];
    }
}

hipError_t launch_chunk_bf16(const bf16 *q, const bf16 *k, const bf16 *v, const bf16 *g,
                             const bf16 *beta, const bf16 *gate, const float *init, bf16 *out,
                             float *final_state, const int32_t *cu, int N, int T, int H,
                             int64_t n_slots, float scale, void *workspace, hipStream_t stream)
{
    static std::once_flag attr_once;
    static hipError_t attr_err = hipSuccess;
    std::call_once(attr_once, [] {
        attr_err = hipFuncSetAttribute(reinterpret_cast<const void *>(kda_prep_bf16_kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(PrepSmem));
    });
    if (attr_err != hipSuccess)
        return attr_err;
    if (n_slots > 0 && H > 0) {
        hipLaunchKernelGGL(kda_prep_bf16_kernel, dim3((unsigned)n_slots, (unsigned)H),
                           dim3(kPrepThreads), sizeof(PrepSmem), stream, q, k, v, g, beta, cu, N,
                           T, H, scale, static_cast<uint8_t *>(workspace));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t units = (int64_t)N * H;
    if (units > 0) {
        const int64_t blocks = (units + 7) / 8 * 8 * kNumVBlocks;
        hipLaunchKernelGGL(kda_chain_bf16_kernel, dim3((unsigned)blocks), dim3(kChainThreads), 0,
                           stream,
                           gate, init, out, final_state, cu, T, H, (int)units,
                           static_cast<const uint8_t *>(workspace));
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
