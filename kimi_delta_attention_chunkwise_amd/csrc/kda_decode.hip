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

// kPro: the prologue bits in `pro` are honoured (a separate instantiation,
// so the plain step carries none of its registers or code)
template <typename T, int DK, int DV, bool kPro>
__global__ __launch_bounds__(256) void kda_decode_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v,
    const T *__restrict__ g, const T *__restrict__ beta, const T *__restrict__ gate,
    float *__restrict__ state, T *__restrict__ out, float scale, unsigned pro)
{
    using Geo = DecodeGeom<T, DK, DV>;
    constexpr int CG = Geo::CG, RG = Geo::RG, RPT = Geo::RPT;
    __shared__ f32x4 red_p[RG][CG];
    __shared__ f32x4 red_s[RG][CG];
    __shared__ float red_kq[RG];
    __shared__ float va[DK], vk[DK], vq[DK];          // exp(g), k, q of this unit
    __shared__ float nrm[2];                           // prologue: 1 / |k|, 1 / |q|

    const int64_t unit = blockIdx.x;                 // n * H + h
    const int tid = threadIdx.x;
    const int cg = tid % CG, rg = tid / CG;
    float *S = state + unit * (int64_t)(DK * DV);
    const T *qu = q + unit * DK, *ku = k + unit * DK, *gu = g + unit * DK;

    f32x4 s_reg[RPT];
#pragma unroll
    for (int m = 0; m < RPT; ++m)
        s_reg[m] = *reinterpret_cast<const f32x4 *>(S + (rg + RG * m) * DV + 4 * cg);
    for (int i = tid; i < DK; i += Geo::NT) {
        const float gx = to_f32(gu[i]);
        va[i] = __expf((kPro && (pro & kProG)) ? log_decay_from(gx) : gx);
        vk[i] = to_f32(ku[i]);
        vq[i] = to_f32(qu[i]);
    }
    __syncthreads();
    if (kPro && (pro & kProQK)) {
        // wave 0 reduces |k|^2 and |q|^2 and rescales the staged vectors
        if (tid < 64) {
            float sk = 0.f, sq = 0.f;
            for (int i = tid; i < DK; i += 64) {
                sk += vk[i] * vk[i];
                sq += vq[i] * vq[i];
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                sk += __shfl_xor(sk, o);
                sq += __shfl_xor(sq, o);
            }
            if (tid == 0) {
                nrm[0] = __builtin_amdgcn_rsqf(sk + kNormEps);
                nrm[1] = __builtin_amdgcn_rsqf(sq + kNormEps);
            }
        }
        __syncthreads();
        for (int i = tid; i < DK; i += Geo::NT) {
            vk[i] *= nrm[0];
            vq[i] *= nrm[1];
        }
        __syncthreads();
    }
    float kk[RPT];
    f32x4 p = {0.f, 0.f, 0.f, 0.f}, sq = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + RG * m;
        const float a = va[row], kr = vk[row], qr = vq[row];
        kk[m] = kr;
        s_reg[m] *= a;                                 // decay the key-channel row
        p += s_reg[m] * kr;                            // prediction for the key
        sq += s_reg[m] * qr;                           // decayed state read by q
        kq += kr * qr;
    }
    red_p[rg][cg] = p;
    red_s[rg][cg] = sq;
    if (cg == 0)
        red_kq[rg] = kq;
    __syncthreads();
    f32x4 P = red_p[0][cg], SQ = red_s[0][cg];
    float KQ = red_kq[0];
#pragma unroll
    for (int r = 1; r < RG; ++r) {
        P += red_p[r][cg];
        SQ += red_s[r][cg];
        KQ += red_kq[r];
    }
    const float b = (kPro && (pro & kProBeta)) ? sigmoidf_(to_f32(beta[unit])) : to_f32(beta[unit]);
    f32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        u[i] = b * (to_f32(v[unit * DV + 4 * cg + i]) - P[i]);   // delta-rule correction
#pragma unroll
    for (int m = 0; m < RPT; ++m) {
        const int row = rg + RG * m;
        __builtin_nontemporal_store(s_reg[m] + kk[m] * u,                  // write
                                    reinterpret_cast<f32x4 *>(S + row * DV + 4 * cg));
    }
    if (rg == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = 4 * cg + i;
            const float o = scale * (SQ[i] + KQ * u[i]);          // read after the write
            out[unit * DV + c] = from_f32<T>(sigmoidf_(to_f32(gate[unit * DV + c])) * o);
        }
    }
}

template <typename T, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const void *g,
                                  const void *beta, const void *gate, float *state, void *out,
                                  int N, int H, float scale, unsigned pro, hipStream_t stream)
{
    using Geo = DecodeGeom<T, DK, DV>;
    const int64_t units = (int64_t)N * H;
    if (units == 0)
        return hipSuccess;
    if (pro)
        hipLaunchKernelGGL((kda_decode_kernel<T, DK, DV, true>), dim3((unsigned)units),
                           dim3(Geo::NT), 0, stream, (const T *)q, (const T *)k, (const T *)v,
                           (const T *)g, (const T *)beta, (const T *)gate, state, (T *)out, scale,
                           pro);
    else
        hipLaunchKernelGGL((kda_decode_kernel<T, DK, DV, false>), dim3((unsigned)units),
                           dim3(Geo::NT), 0, stream, (const T *)q, (const T *)k, (const T *)v,
                           (const T *)g, (const T *)beta, (const T *)gate, state, (T *)out, scale,
                           0u);
    return hipGetLastError();
}

hipError_t launch_decode(const void *q, const void *k, const void *v, const void *g,
                         const void *beta, const void *gate, float *state, void *out, int N,
                         int H, int dk, int dv, float scale, int is_bf16, unsigned pro,
                         hipStream_t stream)
{
    if (dk == 128 && dv == 128)
        return is_bf16 ? launch_decode_t<bf16, 128, 128>(q, k, v, g, beta, gate, state, out, N,
                                                         H, scale, pro, stream)
                       : launch_decode_t<float, 128, 128>(q, k, v, g, beta, gate, state, out,
                                                          N, H, scale, pro, stream);
    if (dk == 16 && dv == 16)
        return is_bf16 ? launch_decode_t<bf16, 16, 16>(q, k, v, g, beta, gate, state, out, N,
                                                       H, scale, pro, stream)
                       : launch_decode_t<float, 16, 16>(q, k, v, g, beta, gate, state, out, N,
                                                        H, scale, pro, stream);
    return hipErrorInvalidValue;
}

}  // namespace kda
