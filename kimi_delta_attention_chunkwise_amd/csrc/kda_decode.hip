// kda_decode.hip -- one O(1) KDA decode step, fused (decay, predict, correct,
// write, read, gate) in a single pass over each state slice.
//
// Source: "Kimi K3 second-pass study ledger" (llm-atlas K3_RESEARCH.md),
// section 1 rows Q04/Q05 (decay and delta-rule write), Q07 (decode keeps an
// O(1) state update), Q08 (output gate); section 8 device row (fused decode).
//
// Per (sequence n, head h) one workgroup owns the dk x dv fp32 slice.  Thread
// (column group cg, row group rg) holds columns 4 cg .. 4 cg + 3 of rows
// rg, rg + RG, ... in registers, so the slice is read once and written once
// with 16-byte accesses; a wave covers two full 512-byte rows per access.
// Because S_new = S~ + k u^T, the readout needs no second pass:
//     S~^T q + (k . q) u = S_new^T q
// so p = S~^T k, S~^T q and k . q are reduced together, u is formed, and the
// new slice is written straight from registers.  The state is streamed: it is
// read once and the new slice is stored with nontemporal stores, which keeps
// the write stream from competing with the reads for cache lines (with plain
// stores this step ran at 63% of HBM peak, with nontemporal ones at 86%).
#include "kda_internal.h"

namespace kda {

template <typename T, int DK, int DV>
struct DecodeGeom {
    static constexpr int CG = DV / 4;                       // float4 column groups
    static constexpr int RG = (256 / CG) < DK ? (256 / CG) : DK;
    static constexpr int NT = CG * RG;                       // threads per workgroup
    static constexpr int RPT = DK / RG;                      // rows per thread
    static_assert(DK % RG == 0, "rows split evenly");
};

// Stage exp(g), k and q of one (sequence, token, head) row in LDS (with the
// prologue, g mapped to the log-decay; k and q as given).  Ends with a barrier.
template <typename T, int DK, int NT, bool kPro>
__device__ __forceinline__ void stage_token(const T *qu, const T *ku, const T *gu, float *va,
                                            float *vk, float *vq, unsigned pro, int tid)
{
    for (int i = tid; i < DK; i += NT) {
        const float gx = to_f32(gu[i]);
        va[i] = __expf((kPro && (pro & kProG)) ? log_decay_from(gx) : gx);
        vk[i] = to_f32(ku[i]);
        vq[i] = to_f32(qu[i]);
    }
    __syncthreads();
}

// The prologue's L2 norms of k and q.  Every reduction of a step is linear
// in k and in q, so the kernels reduce with the token's k and q as given and
// scale afterwards: p and k . q by 1 / |k|, S~^T q and k . q by 1 / |q|, and
// the written row k_r by 1 / |k|.  The squares are summed in a fixed order
// (over the rows rg + RG m of row group rg, m ascending, with fused
// multiply-adds; then over the row groups, rg ascending), which the decode,
// verify and commit kernels share, so that the three form the same 1 / |k|.
__device__ __forceinline__ float sq_acc(float x, float acc) { return __fmaf_rn(x, x, acc); }

template <int RG>
__device__ __forceinline__ float inv_norm(const float *part)
{
    float s = part[0];
#pragma unroll
    for (int r = 1; r < RG; ++r)
        s = __fadd_rn(s, part[r]);
    return __builtin_amdgcn_rsqf(s + kNormEps);
}

// The state update of one row quad, written out so that the decode / verify
// kernel and the commit kernel round identically: decay, then k u^T added
// with one fused multiply-add.
__device__ __forceinline__ f32x4 decay_row(const f32x4 &s, float a)
{
    return f32x4{__fmul_rn(s[0], a), __fmul_rn(s[1], a), __fmul_rn(s[2], a), __fmul_rn(s[3], a)};
}
__device__ __forceinline__ f32x4 write_row(const f32x4 &s, float kr, const f32x4 &u)
{
    return f32x4{__fmaf_rn(kr, u[0], s[0]), __fmaf_rn(kr, u[1], s[1]), __fmaf_rn(kr, u[2], s[2]),
                 __fmaf_rn(kr, u[3], s[3])};
}

// The K draft tokens of a verification, on the state in registers: the
// tokens are staged kVerifyGroup at a time (q, k, exp(g), v, the gate logits
// and beta in LDS: one load phase per group, and no token values held in
// registers beside the state), the reductions of token t go to LDS buffer
// t & 1 (one barrier per token), and each token takes exactly the arithmetic
// of a decode step.
constexpr int kVerifyGroup = 4;

template <typename T, int DK, int DV, bool kPro>
__device__ __forceinline__ void verify_tokens(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, const T *__restrict__ gate,
    T *__restrict__ out, float *__restrict__ u_out, f32x4 *s_reg, int64_t n, int h, int K,
    int H, float scale, unsigned pro, int tid)
{
    using Geo = DecodeGeom<T, DK, DV>;
    constexpr int CG = Geo::CG, RG = Geo::RG, RPT = Geo::RPT, NT = Geo::NT;
    constexpr int kG = kVerifyGroup;
    static_assert(NT % 64 == 0, "whole waves");
    __shared__ float va[kG][DK], vk[kG][DK], vq[kG][DK];
    __shared__ float vv[kG][DV], vz[kG][DV], vbeta[kG];
    __shared__ f32x4 red_p[2][RG][CG];
    __shared__ f32x4 red_s[2][RG][CG];
    __shared__ float red_kq[2][RG];
    __shared__ float red_k2[2][RG], red_q2[2][RG];     // prologue: sums of k^2 and q^2
    const bool qk = kPro && (pro & kProQK);
    const int cg = tid % CG, rg = tid / CG;
    for (int t0 = 0; t0 < K; t0 += kG) {
        const int nt = K - t0 < kG ? K - t0 : kG;
        const int64_t row0 = (n * K + t0) * H + h;   // token t0 + tt is row row0 + tt H
        for (int i = tid; i < nt * DK; i += NT) {
            const int tt = i / DK, c = i % DK;
            const int64_t row = row0 + (int64_t)tt * H;
            const float gx = to_f32(g[row * DK + c]);
            va[tt][c] = __expf((kPro && (pro & kProG)) ? log_decay_from(gx) : gx);
            vk[tt][c] = to_f32(k[row * DK + c]);
            vq[tt][c] = to_f32(q[row * DK + c]);
        }
        for (int i = tid; i < nt * DV; i += NT) {
            const int tt = i / DV, c = i % DV;
            const int64_t row = row0 + (int64_t)tt * H;
            vv[tt][c] = to_f32(v[row * DV + c]);
            vz[tt][c] = to_f32(gate[row * DV + c]);
        }
        if (tid < nt)
            vbeta[tid] = to_f32(beta[row0 + (int64_t)tid * H]);
        __syncthreads();
#pragma unroll
        for (int tt = 0; tt < kG; ++tt) {
            if (tt < nt) {
                const int64_t row = row0 + (int64_t)tt * H;
                const int par = (t0 + tt) & 1;
                f32x4 p = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
                float kq = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const int r = rg + RG * m;
                    const float kr = vk[tt][r], qr = vq[tt][r];
                    s_reg[m] = decay_row(s_reg[m], va[tt][r]);
                    p += s_reg[m] * kr;
                    sq += s_reg[m] * qr;
                    kq += kr * qr;
                    if (qk) {
                        k2 = sq_acc(kr, k2);
                        q2 = sq_acc(qr, q2);
                    }
                }
                red_p[par][rg][cg] = p;
                red_s[par][rg][cg] = sq;
                if (cg == 0) {
                    red_kq[par][rg] = kq;
                    if (qk) {
                        red_k2[par][rg] = k2;
                        red_q2[par][rg] = q2;
                    }
                }
                // buffer par is written again for token t + 2 only after every
                // thread has passed this barrier and the next one
                __syncthreads();
                f32x4 P = red_p[par][0][cg], SQ = red_s[par][0][cg];
                float KQ = red_kq[par][0];
#pragma unroll
                for (int r = 1; r < RG; ++r) {
                    P += red_p[par][r][cg];
                    SQ += red_s[par][r][cg];
                    KQ += red_kq[par][r];
                }
                float ik = 1.f;
                if (qk) {
                    const float iq = inv_norm<RG>(red_q2[par]);
                    ik = inv_norm<RG>(red_k2[par]);
                    P = P * ik;
                    SQ = SQ * iq;
                    KQ = __fmul_rn(__fmul_rn(KQ, ik), iq);
                }
                const float b = (kPro && (pro & kProBeta)) ? sigmoidf_(vbeta[tt]) : vbeta[tt];
                const f32x4 vb = *reinterpret_cast<const f32x4 *>(&vv[tt][4 * cg]);
                f32x4 u;
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    u[i] = b * (vb[i] - P[i]);
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const float kr = vk[tt][rg + RG * m];
                    s_reg[m] = write_row(s_reg[m], qk ? __fmul_rn(kr, ik) : kr, u);
                }
                if (rg == 0) {
                    const f32x4 zb = *reinterpret_cast<const f32x4 *>(&vz[tt][4 * cg]);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int c = 4 * cg + i;
                        const float o = scale * (SQ[i] + KQ * u[i]);
                        out[row * DV + c] = from_f32<T>(sigmoidf_(zb[i]) * o);
                    }
                    if (u_out)
                        *reinterpret_cast<f32x4 *>(u_out + row * DV + 4 * cg) = u;
                }
            }
        }
        if (t0 + kG < K)
            __syncthreads();                           // LDS is restaged for the next group
    }
}

// Decode step (K = 1, state written back) and speculative verification
// (K draft tokens run on the state in registers; the state is left as it was
// and each token's correction u is saved for kda_commit_kernel).  Inputs of
// token t of sequence n, head h are row (n K + t) H + h of the [N, K, H, d]
// tensors.  kPro: the prologue bits in `pro` are honoured (a separate
// instantiation, so the plain step carries none of its registers or code).
// kVerify = false is the plain step: one token, the state written back, no
// corrections saved (K, u_out and write_state are ignored).
template <typename T, int DK, int DV, bool kPro, bool kVerify>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, const T *__restrict__ gate,
    float *__restrict__ state, T *__restrict__ out, float *__restrict__ u_out, int K_arg, int H,
    float scale, unsigned pro, int write_state_arg)
{
    const int K = kVerify ? K_arg : 1;
    const bool write_state = kVerify ? write_state_arg != 0 : true;
    using Geo = DecodeGeom<T, DK, DV>;
    constexpr int CG = Geo::CG, RG = Geo::RG, RPT = Geo::RPT;
    __shared__ f32x4 red_p[RG][CG];
    __shared__ f32x4 red_s[RG][CG];
    __shared__ float red_kq[RG];
    __shared__ float va[DK], vk[DK], vq[DK];          // exp(g), k, q of the current token
    __shared__ float red_k2[RG], red_q2[RG];           // prologue: sums of k^2 and q^2
    const bool qk = kPro && (pro & kProQK);

    const int64_t unit = blockIdx.x;                 // n * H + h
    const int64_t n = unit / H;
    const int h = (int)(unit % H);
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    float *S = state + unit * (int64_t)(DK * DV);

    // A verification only reads the slice, and nontemporal loads stream it past
    // the caches (about 5% faster there); the step, which writes the slice back in
    // place, loads it plainly (nontemporal loads made it about 15% slower).
    f32x4 s_reg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const f32x4 *src = reinterpret_cast<const f32x4 *>(S + (rg + RG * m) * DV + 4 * cg);
        if constexpr (kVerify)
            s_reg[m] = __builtin_nontemporal_load(src);
        else
            s_reg[m] = *src;
    }
    if constexpr (kVerify) {
        verify_tokens<T, DK, DV, kPro>(q, k, v, g, beta, gate, out, u_out, s_reg, n, h, K, H,
                                       scale, pro, tid);
    } else {
    for (int t = 0; t < K; ++t) {
        const int64_t row = (n * K + t) * H + h;
        stage_token<T, DK, Geo::NT, kPro>(q + row * DK, k + row * DK, g + row * DK, va, vk, vq,
                                          pro, tid);
        float kk[RPT];
        f32x4 p = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
        float kq = 0.f, k2 = 0.f, q2 = 0.f;
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int r = rg + RG * m;
            const float kr = vk[r], qr = vq[r];
            kk[m] = kr;
            s_reg[m] = decay_row(s_reg[m], va[r]);     // decay the key-channel row
            p += s_reg[m] * kr;                        // prediction for the key
            sq += s_reg[m] * qr;                       // decayed state read by q
            kq += kr * qr;
            if (qk) {
                k2 = sq_acc(kr, k2);
                q2 = sq_acc(qr, q2);
            }
        }
        red_p[rg][cg] = p;
        red_s[rg][cg] = sq;
        if (cg == 0) {
            red_kq[rg] = kq;
            if (qk) {
                red_k2[rg] = k2;
                red_q2[rg] = q2;
            }
        }
        __syncthreads();
        f32x4 P = red_p[0][cg], SQ = red_s[0][cg];
        float KQ = red_kq[0];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            P += red_p[r][cg];
            SQ += red_s[r][cg];
            KQ += red_kq[r];
        }
        if (qk) {
            const float ik = inv_norm<RG>(red_k2), iq = inv_norm<RG>(red_q2);
            P = P * ik;
            SQ = SQ * iq;
            KQ = __fmul_rn(__fmul_rn(KQ, ik), iq);
#pragma unroll
            for (int m = 0; m < RPT; ++m)
                kk[m] = __fmul_rn(kk[m], ik);
        }
        const float bx = to_f32(beta[row]);
        const float b = (kPro && (pro & kProBeta)) ? sigmoidf_(bx) : bx;
        f32x4 u;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            u[i] = b * (to_f32(v[row * DV + 4 * cg + i]) - P[i]);   // delta-rule correction
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            s_reg[m] = write_row(s_reg[m], kk[m], u);               // write
        if (rg == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int c = 4 * cg + i;
                const float o = scale * (SQ[i] + KQ * u[i]);         // read after the write
                out[row * DV + c] = from_f32<T>(sigmoidf_(to_f32(gate[row * DV + c])) * o);
            }
            if (kVerify && u_out)
                *reinterpret_cast<f32x4 *>(u_out + row * DV + 4 * cg) = u;
        }
        // the next token's staging and reductions overwrite LDS only after the
        // next barrier, which every thread reaches after its reads of this one
    }
    }
    if (write_state) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            __builtin_nontemporal_store(s_reg[m], reinterpret_cast<f32x4 *>(
                                                      S + (rg + RG * m) * DV + 4 * cg));
    }
}

// Commit the first accepted[n] verified tokens of sequence n into its state:
// S <- diag(exp(g_t)) S + k_t u_t^T with the corrections u_t saved by the
// verification, which reproduces the verified states exactly.  Tokens are
// staged kCommitGroup at a time (one load phase and one barrier per group;
// with the prologue, one more for the partial sums of k^2), each with the same
// arithmetic as a staged decode step.
constexpr int kCommitGroup = 4;

template <typename T, int DK, int DV, bool kPro>
__global__ __launch_bounds__(256) void kda_commit_kernel(
    const T *__restrict__ k, const T *__restrict__ g, const float *__restrict__ u,
    const int32_t *__restrict__ accepted, float *__restrict__ state, int K, int H, unsigned pro)
{
    using Geo = DecodeGeom<T, DK, DV>;
    constexpr int CG = Geo::CG, RG = Geo::RG, RPT = Geo::RPT, NT = Geo::NT;
    static_assert(NT % 64 == 0, "whole waves");
    __shared__ float va[kCommitGroup][DK], vk[kCommitGroup][DK];
    __shared__ float red_k2[kCommitGroup][RG];         // prologue: sums of k^2
    const bool qk = kPro && (pro & kProQK);

    const int64_t unit = blockIdx.x;
    const int64_t n = unit / H;
    const int h = (int)(unit % H);
    const int acc_raw = accepted[n];
    const int acc = acc_raw < 0 ? 0 : (acc_raw > K ? K : acc_raw);
    if (acc == 0)
        return;                                        // the whole workgroup leaves together
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    float *S = state + unit * (int64_t)(DK * DV);
    f32x4 s_reg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s_reg[m] = *reinterpret_cast<const f32x4 *>(S + (rg + RG * m) * DV + 4 * cg);
    for (int t0 = 0; t0 < acc; t0 += kCommitGroup) {
        const int nt = acc - t0 < kCommitGroup ? acc - t0 : kCommitGroup;
        const int64_t row0 = (n * K + t0) * H + h;     // token t0 + tt is row row0 + tt H
        for (int i = tid; i < nt * DK; i += NT) {
            const int tt = i / DK, c = i % DK;
            const int64_t row = row0 + (int64_t)tt * H;
            const float gx = to_f32(g[row * DK + c]);
            va[tt][c] = __expf((kPro && (pro & kProG)) ? log_decay_from(gx) : gx);
            vk[tt][c] = to_f32(k[row * DK + c]);
        }
        f32x4 ut[kCommitGroup];
#pragma unroll
        for (int tt = 0; tt < kCommitGroup; ++tt)
            if (tt < nt)
                ut[tt] = *reinterpret_cast<const f32x4 *>(u + (row0 + (int64_t)tt * H) * DV +
                                                          4 * cg);
        __syncthreads();
        if (qk) {
            // the decode step's partial sums of k^2, one per row group
            if (cg == 0) {
#pragma unroll
                for (int tt = 0; tt < kCommitGroup; ++tt) {
                    if (tt < nt) {
                        float k2 = 0.f;
#pragma unroll
                        for (int m = 0; m < RPT; ++m)
                            k2 = sq_acc(vk[tt][rg + RG * m], k2);
                        red_k2[tt][rg] = k2;
                    }
                }
            }
            __syncthreads();
        }
#pragma unroll
        for (int tt = 0; tt < kCommitGroup; ++tt) {
            if (tt < nt) {
                const float ik = qk ? inv_norm<RG>(red_k2[tt]) : 1.f;
#pragma unroll
                for (int m = 0; m < RPT; ++m) {
                    const int r = rg + RG * m;
                    const float kr = qk ? __fmul_rn(vk[tt][r], ik) : vk[tt][r];
                    s_reg[m] = write_row(decay_row(s_reg[m], va[tt][r]), kr, ut[tt]);
                }
            }
        }
        __syncthreads();                               // LDS is restaged for the next group
    }
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        __builtin_nontemporal_store(s_reg[m],
                                    reinterpret_cast<f32x4 *>(S + (rg + RG * m) * DV + 4 * cg));
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const void *gate, float *state, void *out,
                                  float *u_out, int N, int K, int H, float scale, unsigned pro,
                                  int write_state, hipStream_t stream)
{
    using Geo = DecodeGeom<T, DK, DV>;
    const int64_t units = (int64_t)N * H;
    if (units == 0)
        return hipSuccess;
    const bool verify = K != 1 || !write_state || u_out;
#define KDA_LAUNCH(PRO, VER)                                                                      \
    hipLaunchKernelGGL((kda_decode_kernel<T, DK, DV, PRO, VER>), dim3((unsigned)units),           \
                       dim3(Geo::NT), 0, stream, (const T *)q, (const T *)k, (const T *)v,        \
                       (const T *)g, (const T *)beta, (const T *)gate, state, (T *)out, u_out, K, \
                       H, scale, pro, write_state)
    if (pro && verify)
        KDA_LAUNCH(true, true);
    else if (pro)
        KDA_LAUNCH(true, false);
    else if (verify)
        KDA_LAUNCH(false, true);
    else
        KDA_LAUNCH(false, false);
#undef KDA_LAUNCH
    return hipGetLastError();
}

template <typename T, int DK, int DV>
static hipError_t launch_commit_t(const void *k, const void *g, const float *u,
                                  const int32_t *accepted, float *state, int N, int K, int H,
                                  unsigned pro, hipStream_t stream)
{
    using Geo = DecodeGeom<T, DK, DV>;
    const int64_t units = (int64_t)N * H;
    if (units == 0)
        return hipSuccess;
    if (pro)
        hipLaunchKernelGGL((kda_commit_kernel<T, DK, DV, true>), dim3((unsigned)units),
                           dim3(Geo::NT), 0, stream, (const T *)k, (const T *)g, u, accepted,
                           state, K, H, pro);
    else
        hipLaunchKernelGGL((kda_commit_kernel<T, DK, DV, false>), dim3((unsigned)units),
                           dim3(Geo::NT), 0, stream, (const T *)k, (const T *)g, u, accepted,
                           state, K, H, 0u);
    return hipGetLastError();
}

#define KDA_DECODE_DISPATCH(CALL)                                                                 \
    do {                                                                                          \
        if (dk == 128 && dv == 128)                                                               \
            return is_bf16 ? CALL(bf16, 128, 128) : CALL(float, 128, 128);                        \
        if (dk == 16 && dv == 16)                                                                 \
            return is_bf16 ? CALL(bf16, 16, 16) : CALL(float, 16, 16);                            \
        return hipErrorInvalidValue;                                                              \
    } while (0)

hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, float *state, void *out,
                         float *u_out, int N, int K, int H, int dk, int dv, float scale,
                         int is_bf16, unsigned pro, int write_state, hipStream_t stream)
{
#define KDA_CALL(T, DK, DV)                                                                       \
    launch_decode_t<T, DK, DV>(q, k, v, g, beta, gate, state, out, u_out, N, K, H, scale, pro,   \
                               write_state, stream)
    KDA_DECODE_DISPATCH(KDA_CALL);
#undef KDA_CALL
}

hipError_t launch_commit(const void *k, const void *g, const float *u, const int32_t *accepted,
                         float *state, int N, int K, int H, int dk, int dv, int is_bf16,
                         unsigned pro, hipStream_t stream)
{
#define KDA_CALL(T, DK, DV)                                                                       \
    launch_commit_t<T, DK, DV>(k, g, u, accepted, state, N, K, H, pro, stream)
    KDA_DECODE_DISPATCH(KDA_CALL);
#undef KDA_CALL
}

}  // namespace kda
