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
//   A  = strict_lower(diag(beta) [k_r e^{G_r - G_s} k_s]),  P the same with
//        q_r and the diagonal included, times scale
//   T  = (I + A)^-1
//   W  = T diag(beta) (K e^G),  U~ = T diag(beta) V,  U = U~ - W S
//   O  = scale (Q e^G) S + P U,  y = sigmoid(z) O
//   S <- diag(e^{G_end}) S + (K e^{G_end - G})^T U
// Only the products inside A and P need e^{-G}.  Each 16 x 16 block (i, j)
// of A and P is formed with the reference point B_i = G at the end of
// subtile i - 1: rows carry e^{G_r - B_i} (in [e^-80, 1]) and columns carry
// e^{B_i - G_s} (<= e^80 on the diagonal block, <= 1 below it), so every bf16
// operand stays inside the fp32/bf16 exponent range because g >= -5 and a
// subtile is 16 tokens long (5 * 16 = 80 < ln(FLT_MAX) = 88.7).
//
// Two kernels:
//   prep  (one 256-thread workgroup per (chunk slot, head); all chunks in
//          parallel): G, A, P (bf16 MFMA), T (fp32 substitution), W and U~
//          (bf16 MFMA), then the chain's operands as MFMA fragments in the
//          workspace record (layout in kda_internal.h).
//   chain (one wave per (sequence, head, 16-wide value block)): walks the
//          chunks in order with the 128 x 16 fp32 state slice in registers:
//          U = U~ - W S, O = Q~ S + P U, gate, store, S <- dec S + K'^T U.
//          Operands that come from its own accumulators (S, U) are fed back
//          to the MFMA without leaving registers; the prep kernel stores the
//          matching A-operands with their k index permuted to fit.
#include "kda_internal.h"

#include <mutex>

namespace kda {

namespace {

constexpr int kGLd = 132;   // fp32 row stride of the G tile (padding against bank conflicts)
constexpr int kALd = 65;    // fp32 row stride of A and T
constexpr int kPLd = 72;    // bf16 row stride of P
constexpr int kWLd = 136;   // bf16 row stride of -W (reuses the G region)

struct PrepSmem {
    float G[kChunk][kGLd];          // cumulative log-decay; later -W in bf16
    float Bref[4][kDK];             // G at the end of the previous subtile (B_0 = 0)
    float Gend[kDK];
    float beta[kChunk];
    float tot[kDK];
    bf16x8 Xf[16][64];              // B fragments of diag(beta) K e^G
    bf16x8 Vf[16][64];              // B fragments of diag(beta) V
    float A[kChunk][kALd];
    bf16 P[kChunk][kPLd];
    float T[kChunk][kALd];
    float X[3][kSub][kSub + 1];     // block products while inverting
};
static_assert(sizeof(float) * kChunk * kGLd >= sizeof(bf16) * kChunk * kWLd, "W fits in G");

__device__ __forceinline__ bf16x8 load8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }

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

__global__ __launch_bounds__(256) void kda_prep_bf16_kernel(
    const bf16 *__restrict__ q, const bf16 *__restrict__ k, const bf16 *__restrict__ v,
    const bf16 *__restrict__ g, const bf16 *__restrict__ beta, const int32_t *__restrict__ cu,
    int N, int T, int H, float scale, uint8_t *__restrict__ ws)
{
    extern __shared__ __align__(16) uint8_t smem_raw[];
    PrepSmem &sm = *reinterpret_cast<PrepSmem *>(smem_raw);

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
    const int64_t hstride = (int64_t)H * kDK;   // elements between consecutive tokens
    const bf16 *qh = q + (tok0 * H + h) * kDK;
    const bf16 *kh = k + (tok0 * H + h) * kDK;
    const bf16 *vh = v + (tok0 * H + h) * kDV;
    const bf16 *gh = g + (tok0 * H + h) * kDK;

    // ---- phase A: per key channel c, rows 32 hh .. 32 hh + 31 -------------------
    const int c = tid & 127, hh = tid >> 7;
    if (tid < kChunk)
        sm.beta[tid] = tid < len ? (float)beta[(tok0 + tid) * H + h] : 0.f;
    float Gl[32];
    {
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = 32 * hh + i;
            run += r < len ? (float)gh[r * hstride + c] : 0.f;
            Gl[i] = run;
        }
    }
    if (hh == 0)
        sm.tot[c] = Gl[31];
    __syncthreads();
    if (hh == 1) {
        const float t0 = sm.tot[c];
#pragma unroll
        for (int i = 0; i < 32; ++i)
            Gl[i] += t0;
    }
#pragma unroll
    for (int i = 0; i < 32; ++i)
        sm.G[32 * hh + i][c] = Gl[i];
    if (hh == 0) {
        sm.Bref[0][c] = 0.f;
        sm.Bref[1][c] = Gl[15];
        sm.Bref[2][c] = Gl[31];
    } else {
        sm.Bref[3][c] = Gl[15];
        sm.Gend[c] = Gl[31];
    }
    __syncthreads();
    {
        const float gend = sm.Gend[c];
        bf16 kp[32], xb[32], vb[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int r = 32 * hh + i;
            const bool ok = r < len;
            const float kv = ok ? (float)kh[r * hstride + c] : 0.f;
            const float vv = ok ? (float)vh[r * hstride + c] : 0.f;
            const float br = sm.beta[r];
            kp[i] = (bf16)(kv * __expf(gend - Gl[i]));   // K' = K e^{G_end - G}
            xb[i] = (bf16)(br * kv * __expf(Gl[i]));      // diag(beta) K e^G
            vb[i] = (bf16)(br * vv);                      // diag(beta) V
        }
        // K'^T fragment (dk tile c / 16, chunk k-step hh); lane (c % 16) + 16 b holds
        // rows perm_row(hh, b, e) of column c.
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 f;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                f[e] = kp[16 * (e >> 2) + 4 * b + (e & 3)];
            *reinterpret_cast<bf16x8 *>(rec + kOffKP + ((c >> 4) * 2 + hh) * kFragBytes +
                                        ((c & 15) + 16 * b) * 16) = f;
        }
        // B fragments of the W / U~ products: k = chunk row 32 hh + 8 b + e, n = channel.
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            bf16x8 fx, fv;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                fx[e] = xb[8 * b + e];
                fv[e] = vb[8 * b + e];
            }
            sm.Xf[hh * 8 + (c >> 4)][(c & 15) + 16 * b] = fx;
            sm.Vf[hh * 8 + (c >> 4)][(c & 15) + 16 * b] = fv;
        }
    }

    // ---- phase B: wave i forms row block i of A and P, and row tile i of Q~ ----
    {
        const int i = wave, m = lane & 15, b = lane >> 4;
        const int ra = 16 * i + m;
        const bool rok = ra < len;
        bf16x8 kr[4], qr[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int ch = 32 * ks + 8 * b;
            bf16x8 kraw = {}, qraw = {};
            if (rok) {
                kraw = load8(kh + ra * hstride + ch);
                qraw = load8(qh + ra * hstride + ch);
            }
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = __expf(sm.G[ra][ch + e] - sm.Bref[i][ch + e]);
                kr[ks][e] = (bf16)((float)kraw[e] * f);
                qr[ks][e] = (bf16)((float)qraw[e] * f);
            }
        }
        for (int jb = 0; jb <= i; ++jb) {
            const int s = 16 * jb + m;
            const bool sok = s < len;
            f32x4 accA = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int ch = 32 * ks + 8 * b;
                bf16x8 kraw = {};
                if (sok)
                    kraw = load8(kh + s * hstride + ch);
                bf16x8 kc;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    kc[e] = (bf16)((float)kraw[e] * __expf(sm.Bref[i][ch + e] - sm.G[s][ch + e]));
                accA = mfma16(kr[ks], kc, accA);
                accP = mfma16(qr[ks], kc, accP);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * i + 4 * b + e, col = 16 * jb + m;
                const bool below = jb < i || col < row;
                const bool lower = jb < i || col <= row;
                sm.A[row][col] = below ? sm.beta[row] * accA[e] : 0.f;
                sm.P[row][col] = (bf16)(lower ? scale * accP[e] : 0.f);
            }
        }
        for (int jb = i + 1; jb < 4; ++jb) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * i + 4 * b + e, col = 16 * jb + m;
                sm.A[row][col] = 0.f;
                sm.P[row][col] = (bf16)0.f;
                sm.T[row][col] = 0.f;
            }
        }
        // Q~ = scale Q e^G as the chain's A operand: row 16 i + m, k in perm order.
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            bf16x8 f = {};
            if (rok) {
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const int ch = 32 * ks + 16 * half + 4 * b;
                    const bf16x4 qv = *reinterpret_cast<const bf16x4 *>(qh + ra * hstride + ch);
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        f[4 * half + e] = (bf16)(scale * (float)qv[e] * __expf(sm.G[ra][ch + e]));
                }
            }
            *reinterpret_cast<bf16x8 *>(rec + kOffQB + (i * 4 + ks) * kFragBytes + lane * 16) = f;
        }
    }
    __syncthreads();

    // ---- phase C: T = (I + A)^-1 ------------------------------------------------
    if (wave == 0) {
        // diagonal 16 x 16 blocks by forward substitution, one column per lane
        const int blk = lane >> 4, col = lane & 15, o = 16 * blk;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float acc = (r == col) ? 1.f : 0.f;
#pragma unroll
            for (int s = 0; s < r; ++s)
                acc -= sm.A[o + r][o + s] * x[s];
            x[r] = (r < col) ? 0.f : acc;
        }
#pragma unroll
        for (int r = 0; r < 16; ++r)
            sm.T[o + r][o + col] = x[r];
    }
    __syncthreads();
    {
        // off-diagonal blocks: T_ab = -T_aa (sum_{m=b}^{a-1} A_am T_mb), by distance a - b
        const int rr = tid >> 4, cc = tid & 15;
        for (int dist = 1; dist < 4; ++dist) {
            const int nb = 4 - dist;
            for (int p = 0; p < nb; ++p) {
                const int a = p + dist, bb = p;
                float acc = 0.f;
                for (int mm = bb; mm < a; ++mm)
#pragma unroll
                    for (int s = 0; s < 16; ++s)
                        acc += sm.A[16 * a + rr][16 * mm + s] * sm.T[16 * mm + s][16 * bb + cc];
                sm.X[p][rr][cc] = acc;
            }
            __syncthreads();
            for (int p = 0; p < nb; ++p) {
                const int a = p + dist, bb = p;
                float acc = 0.f;
#pragma unroll
                for (int s = 0; s < 16; ++s)
                    acc -= sm.T[16 * a + rr][16 * a + s] * sm.X[p][s][cc];
                sm.T[16 * a + rr][16 * bb + cc] = acc;
            }
            __syncthreads();
        }
    }

    // ---- phase D: W = T X and U~ = T V (bf16 MFMA, fp32 accumulate) ----------
    {
        const int m = lane & 15, b = lane >> 4;
        bf16x8 tf[4][2];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks) {
                bf16x8 f = {};
                if (ks <= (mt >> 1)) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        f[e] = (bf16)sm.T[16 * mt + m][32 * ks + 8 * b + e];
                }
                tf[mt][ks] = f;
            }
        bf16 *sW = reinterpret_cast<bf16 *>(&sm.G[0][0]);
#pragma unroll
        for (int q2 = 0; q2 < 2; ++q2) {
            const int nt = 2 * wave + q2;
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                f32x4 accW = {0.f, 0.f, 0.f, 0.f}, accU = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < 2; ++ks) {
                    if (ks <= (mt >> 1)) {
                        accW = mfma16(tf[mt][ks], sm.Xf[ks * 8 + nt][lane], accW);
                        accU = mfma16(tf[mt][ks], sm.Vf[ks * 8 + nt][lane], accU);
                    }
                }
                bf16x4 u4;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    u4[e] = (bf16)accU[e];
                    sW[(16 * mt + 4 * b + e) * kWLd + 16 * nt + m] = (bf16)(-accW[e]);
                }
                *reinterpret_cast<bf16x4 *>(rec + kOffUT + nt * 2048 + lane * 32 + mt * 8) = u4;
            }
        }
    }
    __syncthreads();

    // ---- phase E: -W and P as the chain's A-operand fragments, and e^{G_end} ----
    {
        const bf16 *sW = reinterpret_cast<const bf16 *>(&sm.G[0][0]);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int it = tid + 256 * x, f = it >> 6, L = it & 63;
            const int mt = f >> 2, ks = f & 3, row = 16 * mt + (L & 15), bb = L >> 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(sW + row * kWLd + 32 * ks + 4 * bb);
            const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(sW + row * kWLd + 32 * ks + 16 + 4 * bb);
            bf16x8 o = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<bf16x8 *>(rec + kOffWN + f * kFragBytes + L * 16) = o;
        }
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const int it = tid + 256 * x, f = it >> 6, L = it & 63;
            const int mt = f >> 1, ks = f & 1, row = 16 * mt + (L & 15), bb = L >> 4;
            const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(&sm.P[row][32 * ks + 4 * bb]);
            const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(&sm.P[row][32 * ks + 16 + 4 * bb]);
            bf16x8 o = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            *reinterpret_cast<bf16x8 *>(rec + kOffPP + f * kFragBytes + L * 16) = o;
        }
        if (tid < kDK)
            reinterpret_cast<float *>(rec + kOffDEC)[tid] = __expf(sm.Gend[tid]);
    }
}

__global__ __launch_bounds__(64) void kda_chain_bf16_kernel(
    const bf16 *__restrict__ gate, const float *__restrict__ init, bf16 *__restrict__ out,
    float *__restrict__ final_state, const int32_t *__restrict__ cu, int T, int H,
    const uint8_t *__restrict__ ws)
{
    const int blk = blockIdx.x % kNumVBlocks;
    const int64_t unit = blockIdx.x / kNumVBlocks;          // n * H + h
    const int n = (int)(unit / H), h = (int)(unit % H);
    const int lane = threadIdx.x, m = lane & 15, b = lane >> 4;
    const SeqInfo si = seq_info(cu, n, T, kChunk);
    const int col = kVBlock * blk + m;
    const int64_t sbase = unit * (int64_t)(kDK * kDV);

    // state slice: tile t holds rows 16 t + 4 b + i, column col
    f32x4 S[8];
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            S[t][i] = init ? init[sbase + (16 * t + 4 * b + i) * kDV + col] : 0.f;

    const int64_t nch = (si.len + kChunk - 1) / kChunk;
    for (int64_t jc = 0; jc < nch; ++jc) {
        const uint8_t *rec = ws + ((si.slot0 + jc) * H + h) * (int64_t)kRecBytes;
        const bf16x8 *WN = reinterpret_cast<const bf16x8 *>(rec + kOffWN) + lane;
        const bf16x8 *QB = reinterpret_cast<const bf16x8 *>(rec + kOffQB) + lane;
        const bf16x8 *KP = reinterpret_cast<const bf16x8 *>(rec + kOffKP) + lane;
        const bf16x8 *PP = reinterpret_cast<const bf16x8 *>(rec + kOffPP) + lane;
        const bf16x8 ut_lo = *reinterpret_cast<const bf16x8 *>(rec + kOffUT + blk * 2048 + lane * 32);
        const bf16x8 ut_hi = *reinterpret_cast<const bf16x8 *>(rec + kOffUT + blk * 2048 + lane * 32 + 16);

        bf16x8 Sb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Sb[ks][e] = (bf16)S[2 * ks][e];
                Sb[ks][4 + e] = (bf16)S[2 * ks + 1][e];
            }
        // U = U~ - W S
        f32x4 U[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                U[t][e] = (float)((t < 2) ? ut_lo[4 * t + e] : ut_hi[4 * (t - 2) + e]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                U[t] = mfma16(WN[(t * 4 + ks) * 64], Sb[ks], U[t]);
        // O = Q~ S + P U
        f32x4 O[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            O[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                O[t] = mfma16(QB[(t * 4 + ks) * 64], Sb[ks], O[t]);
        }
        bf16x8 Ub[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                Ub[ks][e] = (bf16)U[2 * ks][e];
                Ub[ks][4 + e] = (bf16)U[2 * ks + 1][e];
            }
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                O[t] = mfma16(PP[(t * 2 + ks) * 64], Ub[ks], O[t]);
        // S <- diag(e^{G_end}) S + K'^T U
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const f32x4 d = *reinterpret_cast<const f32x4 *>(rec + kOffDEC + (16 * t + 4 * b) * 4);
            S[t] *= d;
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
                S[t] = mfma16(KP[(t * 2 + ks) * 64], Ub[ks], S[t]);
        }
        // output gate and store
        const int64_t tok0 = si.bos + jc * kChunk;
        const int64_t lenc = si.len - jc * kChunk;
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int row = 16 * t + 4 * b + e;
                if (row < lenc) {
                    const int64_t o = ((tok0 + row) * H + h) * kDV + col;
                    out[o] = (bf16)(sigmoidf_((float)gate[o]) * O[t][e]);
                }
            }
    }
    if (final_state) {
#pragma unroll
        for (int t = 0; t < 8; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                final_state[sbase + (16 * t + 4 * b + i) * kDV + col] = S[t][i];
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
        hipLaunchKernelGGL(kda_prep_bf16_kernel, dim3((unsigned)n_slots, (unsigned)H), dim3(256),
                           sizeof(PrepSmem), stream, q, k, v, g, beta, cu, N, T, H, scale,
                           static_cast<uint8_t *>(workspace));
        hipError_t e = hipGetLastError();
        if (e != hipSuccess)
            return e;
    }
    const int64_t chains = (int64_t)N * H * kNumVBlocks;
    if (chains > 0) {
        hipLaunchKernelGGL(kda_chain_bf16_kernel, dim3((unsigned)chains), dim3(64), 0, stream,
                           gate, init, out, final_state, cu, T, H,
                           static_cast<const uint8_t *>(workspace));
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace kda
