// kda_chunk_f32.hip -- chunkwise KDA forward in fp32 for small heads
// (dk = dv = 16, 16-token chunks).
//
// Source: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
// section 1 row Q07 (state passed recurrently between chunks, dense matrix
// work inside a chunk) and row Q06 (g >= -5, so inside a 16-token chunk the
// reciprocal of the cumulative decay is at most exp(80), finite in fp32);
// "Kimi K3 report reveals training and systems stack" (16-token tiles).
//
// One workgroup of 256 threads per (sequence, head); thread (r, c) owns
// element (r, c) of every 16 x 16 matrix of the chunk.  Per chunk, with G the
// inclusive cumulative log-decay from the chunk start:
//   A  = strict_lower(diag(beta) (K e^G)(K e^-G)^T)
//   P  = lower_incl((Q e^G)(K e^-G)^T) * scale
//   T  = (I + A)^-1                      (forward substitution, 16 columns)
//   W  = T diag(beta) (K e^G),   U~ = T diag(beta) V,   U = U~ - W S
//   O  = scale (Q e^G) S + P U,  y = sigmoid(z) O
//   S <- diag(e^{G_end}) S + (K e^{G_end - G})^T U
// All arithmetic is fp32.
#include "kda_internal.h"

namespace kda {

namespace {
constexpr int D = 16;      // dk = dv = chunk
constexpr int LD = D + 1;  // padded LDS row
}  // namespace

__global__ __launch_bounds__(256) void kda_chunk_f32_kernel(
    const float *__restrict__ q, const float *__restrict__ k, const float *__restrict__ v,
    const float *__restrict__ g, const float *__restrict__ beta, const float *__restrict__ gate,
    const float *__restrict__ init, float *__restrict__ out, float *__restrict__ final_state,
    float *__restrict__ snaps, int snap_interval, const int32_t *__restrict__ cu, int T, int H,
    float scale, unsigned pro)
{
    __shared__ float sS[D][LD], sG[D][LD], sQb[D][LD], sKb[D][LD], sKc[D][LD], sKp[D][LD];
    __shared__ float sX[D][LD], sVb[D][LD], sA[D][LD], sP[D][LD], sT[D][LD], sW[D][LD];
    __shared__ float sU[D][LD], sBeta[D];

    const int unit = blockIdx.x;             // n * H + h
    const int n = unit / H, h = unit % H;
    const int tid = threadIdx.x;
    const int r = tid / D, c = tid % D;
    const SeqInfo si = seq_info(cu, n, T, D);

    sS[r][c] = init ? init[(int64_t)unit * D * D + r * D + c] : 0.f;

    for (int64_t c0 = 0; c0 < si.len; c0 += D) {
        const int L = (int)((si.len - c0) < D ? (si.len - c0) : D);
        const bool valid = r < L;
        const int64_t tok = si.bos + c0 + r;
        const int64_t off = (tok * H + h) * D + c;
        float qv = valid ? q[off] : 0.f;
        float kv = valid ? k[off] : 0.f;
        const float vv = valid ? v[off] : 0.f;
        const float zv = valid ? gate[off] : 0.f;
        const float gx = valid ? g[off] : 0.f;
        sG[r][c] = valid && (pro & kProG) ? log_decay_from(gx) : gx;
        if (c == 0) {
            const float bx = valid ? beta[tok * H + h] : 0.f;
            sBeta[r] = valid && (pro & kProBeta) ? sigmoidf_(bx) : bx;
        }
        if (pro & kProQK) {
            // row r lives in 16 consecutive lanes: reduce q^2 and k^2 across them
            float sq = qv * qv, sk = kv * kv;
#pragma unroll
            for (int o = 8; o >= 1; o >>= 1) {
                sq += __shfl_xor(sq, o, D);
                sk += __shfl_xor(sk, o, D);
            }
            qv *= __builtin_amdgcn_rsqf(sq + kNormEps);
            kv *= __builtin_amdgcn_rsqf(sk + kNormEps);
        }
        __syncthreads();
        float Gr = 0.f;
        for (int u = 0; u <= r; ++u)
            Gr += sG[u][c];
        float Gend = 0.f;
        for (int u = 0; u < D; ++u)
            Gend += sG[u][c];
        const float br = sBeta[r];
        __syncthreads();
        sQb[r][c] = scale * qv * expf(Gr);
        sKb[r][c] = kv * expf(Gr);
        sKc[r][c] = kv * expf(-Gr);
        sKp[r][c] = kv * expf(Gend - Gr);
        sX[r][c] = br * kv * expf(Gr);
        sVb[r][c] = br * vv;
        sG[r][c] = Gend;                      // row r now holds G_end for channel c
        __syncthreads();
        float a = 0.f, p = 0.f;
        for (int j = 0; j < D; ++j) {
            a += sKb[r][j] * sKc[c][j];
            p += sQb[r][j] * sKc[c][j];
        }
        sA[r][c] = (c < r) ? br * a : 0.f;
        sP[r][c] = (c <= r) ? p : 0.f;
        __syncthreads();
        if (tid < D) {                        // column tid of (I + A)^-1
            // x[s] = 0 for s < tid, so the full-range sums below add only zeros there
            float x[D];
#pragma unroll
            for (int i = 0; i < D; ++i) {
                float acc = (i == tid) ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < i; ++s)
                    acc -= sA[i][s] * x[s];
                x[i] = (i < tid) ? 0.f : acc;
            }
#pragma unroll
            for (int i = 0; i < D; ++i)
                sT[i][tid] = x[i];
        }
        __syncthreads();
        float w = 0.f, ut = 0.f;
        for (int s = 0; s <= r; ++s) {
            w += sT[r][s] * sX[s][c];
            ut += sT[r][s] * sVb[s][c];
        }
        sW[r][c] = w;
        __syncthreads();
        float ws = 0.f;
        for (int j = 0; j < D; ++j)
            ws += sW[r][j] * sS[j][c];
        sU[r][c] = ut - ws;
        __syncthreads();
        float o = 0.f;
        for (int j = 0; j < D; ++j)
            o += sQb[r][j] * sS[j][c];
        for (int s = 0; s <= r; ++s)
            o += sP[r][s] * sU[s][c];
        if (valid)
            out[(tok * H + h) * D + c] = (1.0f / (1.0f + expf(-zv))) * o;
        float sn = expf(sG[0][r]) * sS[r][c];   // G_end of key channel r
        for (int s = 0; s < D; ++s)
            sn += sKp[s][r] * sU[s][c];
        __syncthreads();
        sS[r][c] = sn;
        // snapshot of the state after the first c0 + L tokens
        const int64_t pos = c0 + L;
        if (snaps && pos % snap_interval == 0) {
            const int64_t slot = snap_slot0(cu, n, T, snap_interval) + pos / snap_interval - 1;
            snaps[(slot * H + h) * D * D + r * D + c] = sn;
        }
        __syncthreads();
    }
    __syncthreads();
    if (final_state)
        final_state[(int64_t)unit * D * D + r * D + c] = sS[r][c];
}

hipError_t launch_chunk_f32(const float *q, const float *k, const float *v, const float *g,
                            const float *beta, const float *gate, const float *init, float *out,
                            float *final_state, float *snaps, int snap_interval,
                            const int32_t *cu, int N, int T, int H, float scale, unsigned pro,
                            hipStream_t stream)
{
    const int64_t units = (int64_t)N * H;
    if (units == 0)
        return hipSuccess;
    hipLaunchKernelGGL(kda_chunk_f32_kernel, dim3((unsigned)units), dim3(256), 0, stream, q, k,
                       v, g, beta, gate, init, out, final_state, snaps, snap_interval, cu, T, H,
                       scale, pro);
    return hipGetLastError();
}

}  // namespace kda
