// kda_chunk_bwd_f32.hip -- chunkwise KDA backward, fp32 arithmetic,
// dk = dv = 16, 16-token chunks.
//
// Source: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
// section 1 row Q07 (the chunkwise form serves training as well as prefill:
// the state is passed recurrently between chunks, dense matrix work inside a
// chunk) and row Q06 (g >= -5 bounds the cumulative decay inside a 16-token
// chunk by exp(80)).
//
// One chunk with entry state S, in the "U form" (r, s rows of the chunk, G
// the within-chunk cumulative log-decay including the row itself, Ge = G of
// the last row, B = G of row 7, the midpoint reference of the pair products):
//   Qs = scale Q e^G,  Ks = K e^G,  Kp = K e^{Ge - G}        (factors <= 1)
//   Qr = scale Q e^{G-B},  Kr = K e^{G-B},  Kc = K e^{B-G}    (within e^+-40)
//   A  = strict_lower(diag(beta) Kr Kc^T),  T = (I + A)^-1
//   P  = lower_incl(Qr Kc^T)
//   W  = T diag(beta) Ks,  U~ = T diag(beta) V,  U = U~ - W S
//   O  = Qs S + P U,  Y = sigmoid(Z) O,  S' = diag(e^Ge) S + Kp^T U
// The backward walks the chunks in reverse with dS' (the gradient of the
// state leaving the chunk):
//   dO = dY sigmoid(Z),  dZ = dY O sigmoid'(Z)
//   dU = Kp dS' + P^T dO,  dKp = U dS'^T,  dQs = dO S^T,  dP = lower_incl(dO U^T)
//   dW = -dU S^T,  dS = diag(e^Ge) dS' + Qs^T dO - W^T dU
//   dT = dW (diag(beta) Ks)^T + dU (diag(beta) V)^T,  dA = strict_lower(-T^T dT T^T)
//   dKs = diag(beta) T^T dW,  dV = diag(beta) T^T dU
//   dKr = diag(beta) dA Kc,  dKc = dA^T diag(beta) Kr + dP^T Qr,  dQr = dP Kc
//   dbeta = rowsum((T^T dW) Ks + (T^T dU) V + dA (Kr Kc^T))
//   dQ = scale (e^G dQs + e^{G-B} dQr),
//   dK = e^G dKs + e^{G-B} dKr + e^{B-G} dKc + e^{Ge-G} dKp
//   dG = dQs Qs + dQr Qr + dKs Ks + dKr Kr - dKc Kc - dKp Kp
//   dGe = colsum(dKp Kp) + e^Ge rowsum(dS' S),  dg_u = sum_{r >= u} dG_r + dGe
// The reference B cancels inside A and P, so the loss does not depend on it
// and it carries no gradient.  Entry states come from a forward pass over the
// sequence in the same kernel and are kept in the workspace, one 16 x 16 fp32
// slice per (chunk slot, head).
#include "kda_internal.h"

namespace kda {

namespace {

constexpr int D = 16;
constexpr int LD = D + 1;
constexpr int kRef = 7;   // row whose cumulative decay is the pair-product reference

typedef float Mat[D][LD];

// Column `col` of (I + A)^-1 for strictly lower A, by forward substitution.
__device__ __forceinline__ void inverse_column(const Mat &A, Mat &T, int col)
{
    float x[D];
#pragma unroll
    for (int i = 0; i < D; ++i) {
        float acc = (i == col) ? 1.f : 0.f;
#pragma unroll
        for (int s = 0; s < i; ++s)
            acc -= A[i][s] * x[s];
        x[i] = acc;
    }
#pragma unroll
    for (int i = 0; i < D; ++i)
        T[i][col] = x[i];
}

struct Factors {
    float eg, egb, ebg, ep;   // e^G, e^{G-B}, e^{B-G}, e^{Ge-G} of one element
};

}  // namespace

__global__ __launch_bounds__(256) void kda_chunk_bwd_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ gate,
    const float *__restrict__ init, const float *__restrict__ dout,
    const float *__restrict__ dfinal, float *__restrict__ dq, float *__restrict__ dk,
    float *__restrict__ dv, float *__restrict__ dg, float *__restrict__ dbeta,
    float *__restrict__ dgate, float *__restrict__ dinit, const int32_t *__restrict__ cu, int T,
    int H, float scale, float *__restrict__ ws)
{
    __shared__ Mat sS, sdS, sV, sQs, sKs, sKp, sQr, sKr, sKc;
    __shared__ Mat sM, sA, sP, sT, sW, sU, sdO, sdU, sdW, sdP, sdT, sdA, sX;
    __shared__ float sBeta[D], sDec[D], sdGe[D];

    const int unit = blockIdx.x;             // n * H + h
    const int n = unit / H, h = unit % H;
    const int tid = threadIdx.x;
    const int r = tid / D, c = tid % D;
    const SeqInfo si = seq_info(cu, n, T, D);
    const int64_t nch = (si.len + D - 1) / D;
    // entry state of chunk j: [slot][H][D][D]
    auto wstate = [&](int64_t j) { return ws + ((si.slot0 + j) * H + h) * (int64_t)(D * D); };

    // Loads chunk c0 .. c0 + L - 1 (rows past L read as zero, and g = 0 there
    // keeps G constant) and forms the factored operands; returns this
    // thread's exponent factors for element (r, c).
    auto load_chunk = [&](int64_t c0, int L) -> Factors {
        const bool valid = r < L;
        const int64_t off = ((si.bos + c0 + r) * H + h) * D + c;
        const float qv = valid ? q[off] : 0.f, kv = valid ? k[off] : 0.f;
        sV[r][c] = valid ? v[off] : 0.f;
        sX[r][c] = valid ? g[off] : 0.f;
        if (c == 0)
            sBeta[r] = valid ? beta[(si.bos + c0 + r) * H + h] : 0.f;
        __syncthreads();
        float G = 0.f, Ge = 0.f, Bref = 0.f;
        for (int u = 0; u < D; ++u) {
            const float x = sX[u][c];
            Ge += x;
            if (u <= r)
                G += x;
            if (u <= kRef)
                Bref += x;
        }
        Factors f;
        f.eg = expf(G);
        f.egb = expf(G - Bref);
        f.ebg = expf(Bref - G);
        f.ep = expf(Ge - G);
        sQs[r][c] = scale * qv * f.eg;
        sKs[r][c] = kv * f.eg;
        sKp[r][c] = kv * f.ep;
        sQr[r][c] = scale * qv * f.egb;
        sKr[r][c] = kv * f.egb;
        sKc[r][c] = kv * f.ebg;
        if (r == 0)
            sDec[c] = expf(Ge);
        __syncthreads();
        return f;
    };

    // A (and, for the backward, the unmasked M = Kr Kc^T and P), then T, W, U.
    auto chunk_core = [&](bool backward) {
        float m = 0.f;
        for (int x = 0; x < D; ++x)
            m += sKr[r][x] * sKc[c][x];
        sA[r][c] = (c < r) ? sBeta[r] * m : 0.f;
        if (backward) {
            float p = 0.f;
            for (int x = 0; x < D; ++x)
                p += sQr[r][x] * sKc[c][x];
            sM[r][c] = m;
            sP[r][c] = (c <= r) ? p : 0.f;
        }
        __syncthreads();
        if (tid < D)
            inverse_column(sA, sT, tid);
        __syncthreads();
        float w = 0.f, ut = 0.f;
        for (int s = 0; s <= r; ++s) {
            w += sT[r][s] * sBeta[s] * sKs[s][c];
            ut += sT[r][s] * sBeta[s] * sV[s][c];
        }
        sW[r][c] = w;
        __syncthreads();
        for (int x = 0; x < D; ++x)
            ut -= sW[r][x] * sS[x][c];
        sU[r][c] = ut;
        __syncthreads();
    };

    // ---------------- forward: the entry state of every chunk ----------------
    sS[r][c] = init ? init[(int64_t)unit * D * D + r * D + c] : 0.f;
    __syncthreads();
    for (int64_t j = 0; j < nch; ++j) {
        const int64_t c0 = j * D;
        const int L = (int)((si.len - c0) < D ? (si.len - c0) : D);
        wstate(j)[r * D + c] = sS[r][c];
        load_chunk(c0, L);
        chunk_core(false);
        float sn = sDec[r] * sS[r][c];
        for (int s = 0; s < D; ++s)
            sn += sKp[s][r] * sU[s][c];
        __syncthreads();
        sS[r][c] = sn;
        __syncthreads();
    }

    // ---------------- backward over the chunks, last to first ----------------
    sdS[r][c] = dfinal ? dfinal[(int64_t)unit * D * D + r * D + c] : 0.f;
    for (int64_t j = nch - 1; j >= 0; --j) {
        const int64_t c0 = j * D;
        const int L = (int)((si.len - c0) < D ? (si.len - c0) : D);
        const bool valid = r < L;
        const int64_t tok = si.bos + c0 + r;
        const int64_t off = (tok * H + h) * D + c;
        sS[r][c] = wstate(j)[r * D + c];   // written by this same thread in the forward
        const Factors f = load_chunk(c0, L);
        chunk_core(true);
        const float br = sBeta[r];

        // output and gate
        float o = 0.f;
        for (int x = 0; x < D; ++x)
            o += sQs[r][x] * sS[x][c];
        for (int s = 0; s <= r; ++s)
            o += sP[r][s] * sU[s][c];
        const float z = valid ? gate[off] : 0.f;
        const float dy = valid ? dout[off] : 0.f;
        const float sg = 1.f / (1.f + expf(-z));
        if (valid)
            dgate[off] = dy * o * sg * (1.f - sg);
        sdO[r][c] = dy * sg;
        __syncthreads();

        // O = Qs S + P U and S' = diag(e^Ge) S + Kp^T U
        float dU = 0.f, dKp = 0.f, dQs = 0.f, dP = 0.f;
        for (int x = 0; x < D; ++x) {
            dU += sKp[r][x] * sdS[x][c];
            dKp += sU[r][x] * sdS[c][x];
            dQs += sdO[r][x] * sS[c][x];
        }
        for (int s = r; s < D; ++s)
            dU += sP[s][r] * sdO[s][c];
        if (c <= r)
            for (int x = 0; x < D; ++x)
                dP += sdO[r][x] * sU[c][x];
        if (r == 0) {
            float acc = 0.f;
            for (int x = 0; x < D; ++x)
                acc += sdS[c][x] * sS[c][x];
            sdGe[c] = sDec[c] * acc;
        }
        sdU[r][c] = dU;
        sdP[r][c] = dP;
        __syncthreads();

        // U = U~ - W S; the state gradient on entry to the chunk; P = Qr Kc^T
        float dW = 0.f, dSin = sDec[r] * sdS[r][c];
        for (int x = 0; x < D; ++x) {
            dW -= sdU[r][x] * sS[c][x];
            dSin += sQs[x][r] * sdO[x][c] - sW[x][r] * sdU[x][c];
        }
        float dQr = 0.f;
        for (int s = 0; s <= r; ++s)
            dQr += sdP[r][s] * sKc[s][c];
        sdW[r][c] = dW;
        __syncthreads();

        // W = T diag(beta) Ks and U~ = T diag(beta) V
        float dT = 0.f, tdw = 0.f, tdu = 0.f;
        for (int x = 0; x < D; ++x)
            dT += sBeta[c] * (sdW[r][x] * sKs[c][x] + sdU[r][x] * sV[c][x]);
        for (int s = r; s < D; ++s) {
            tdw += sT[s][r] * sdW[s][c];
            tdu += sT[s][r] * sdU[s][c];
        }
        sdT[r][c] = dT;
        __syncthreads();

        // T = (I + A)^-1: dA = strict_lower(-T^T dT T^T)
        float m1 = 0.f;
        for (int s = r; s < D; ++s)
            m1 += sT[s][r] * sdT[s][c];
        sX[r][c] = m1;
        __syncthreads();
        float da = 0.f;
        for (int x = 0; x <= c; ++x)
            da += sX[r][x] * sT[c][x];
        sdA[r][c] = (c < r) ? -da : 0.f;
        __syncthreads();

        // A = strict_lower(diag(beta) Kr Kc^T), P = lower_incl(Qr Kc^T)
        float dKr = 0.f, dKc = 0.f;
        for (int s = 0; s < r; ++s)
            dKr += sdA[r][s] * sKc[s][c];
        dKr *= br;
        for (int r2 = r + 1; r2 < D; ++r2)
            dKc += sdA[r2][r] * sBeta[r2] * sKr[r2][c];
        for (int r2 = r; r2 < D; ++r2)
            dKc += sdP[r2][r] * sQr[r2][c];
        const float dKs = br * tdw;
        if (valid)
            dv[off] = br * tdu;
        float pb = tdw * sKs[r][c] + tdu * sV[r][c] + sdA[r][c] * sM[r][c];
        for (int o2 = D / 2; o2 >= 1; o2 >>= 1)
            pb += __shfl_xor(pb, o2, D);
        if (c == 0 && valid)
            dbeta[tok * H + h] = pb;

        // exponent factors
        if (valid) {
            dq[off] = scale * (f.eg * dQs + f.egb * dQr);
            dk[off] = f.eg * dKs + f.egb * dKr + f.ebg * dKc + f.ep * dKp;
        }
        const float dG = dQs * sQs[r][c] + dQr * sQr[r][c] + dKs * sKs[r][c] +
                         dKr * sKr[r][c] - dKc * sKc[r][c] - dKp * sKp[r][c];
        const float kpdkp = dKp * sKp[r][c];
        __syncthreads();
        sX[r][c] = dG;
        sdT[r][c] = kpdkp;
        __syncthreads();
        float dGe = sdGe[c];
        for (int x = 0; x < D; ++x)
            dGe += sdT[x][c];
        float dgv = dGe;
        for (int x = r; x < D; ++x)
            dgv += sX[x][c];
        if (valid)
            dg[off] = dgv;
        sdS[r][c] = dSin;
        __syncthreads();
    }
    if (dinit)
        dinit[(int64_t)unit * D * D + r * D + c] = sdS[r][c];
}

hipError_t launch_chunk_bwd_f32(const float *q, const float *k, const float *v, const float *g,
                                const float *beta, const float *gate, const float *init,
                                const float *dout, const float *dfinal, float *dq, float *dk,
                                float *dv, float *dg, float *dbeta, float *dgate, float *dinit,
                                const int32_t *cu, int N, int T, int H, float scale, float *ws,
                                hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    if (units == 0)
        return hipSuccess;
    hipLaunchKernelGGL(kda_chunk_bwd_f32_kernel, dim3((unsigned)units), dim3(256), 0, stream, q,
                       k, v, g, beta, gate, init, dout, dfinal, dq, dk, dv, dg, dbeta, dgate,
                       dinit, cu, T, H, scale, ws);
    return hipGetLastError();
}

}  // namespace kda
