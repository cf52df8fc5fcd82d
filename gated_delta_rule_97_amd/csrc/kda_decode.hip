// KDA decode step for gfx950: one token for each of N independent
// sequences, the fp32 state updated in place (Kimi K3 architecture blog
// post, serving-stack section: the recurrent state is updated in place).
//
// Per (sequence, head), with S (dk x dv) row-major in HBM:
//   S' = Diag(e^g) S;  w = S'^T k;  y = S'^T q;  u = beta (v - w)
//   S  = S' + k u^T;   o = S^T q = y + (k . q) u
// The state is streamed through HBM exactly once each way: every thread
// loads its float4 slices of S, the two reductions over dk go through LDS,
// and the updated slices are written back from registers.  This kernel is
// bound by HBM bandwidth (about 0.86 flop per byte at dk = dv = 128).
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

template <class T, int DK, int DV>
__global__ __launch_bounds__(256) void kda_decode_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                        const T *__restrict__ v, const float *__restrict__ g,
                                                        const float *__restrict__ beta, float *__restrict__ state,
                                                        T *__restrict__ o) {
    constexpr int CG = DV / 4;      // float4 column groups
    constexpr int RG = 256 / CG;    // row groups
    constexpr int RPT = DK / RG;    // rows per thread
    static_assert(RG * CG == 256 && RPT * RG == DK, "decode thread split");
    __shared__ float sk[DK], sq[DK], sd[DK];
    __shared__ float4 sw[RG][CG], sy[RG][CG];
    __shared__ float skq;

    const size_t ch = blockIdx.x;  // sequence * H + head
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    float *S = state + ch * DK * DV;

    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)  // rows i*RG + rg: a workgroup-wide load is one contiguous span
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);
    for (int c = tid; c < DK; c += 256) {
        sk[c] = to_f32(k[ch * DK + c]);
        sq[c] = to_f32(q[ch * DK + c]);
        sd[c] = exp_e(g[ch * DK + c]);
    }
    __syncthreads();
    if (tid < 64) {
        float p = 0.f;
        for (int c = tid; c < DK; c += 64) p += sk[c] * sq[c];
#pragma unroll
        for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (tid == 0) skq = p;
    }
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f), y = w;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = i * RG + rg;
        const float f = sd[c], kc = sk[c], qc = sq[c];
        s[i] *= f;
        w.x += kc * s[i][0]; w.y += kc * s[i][1]; w.z += kc * s[i][2]; w.w += kc * s[i][3];
        y.x += qc * s[i][0]; y.y += qc * s[i][1]; y.z += qc * s[i][2]; y.w += qc * s[i][3];
    }
    sw[rg][cg] = w;
    sy[rg][cg] = y;
    __syncthreads();
    float4 W = make_float4(0.f, 0.f, 0.f, 0.f), Y = W;
#pragma unroll
    for (int r = 0; r < RG; ++r) {
        const float4 a = sw[r][cg], b = sy[r][cg];
        W.x += a.x; W.y += a.y; W.z += a.z; W.w += a.w;
        Y.x += b.x; Y.y += b.y; Y.z += b.z; Y.w += b.w;
    }
    const float bt = beta[ch];
    const T *vp = v + ch * DV + 4 * cg;
    float4 u;
    u.x = bt * (to_f32(vp[0]) - W.x);
    u.y = bt * (to_f32(vp[1]) - W.y);
    u.z = bt * (to_f32(vp[2]) - W.z);
    u.w = bt * (to_f32(vp[3]) - W.w);
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = i * RG + rg;
        const float kc = sk[c];
        floatx4 r = s[i];
        r[0] += kc * u.x; r[1] += kc * u.y; r[2] += kc * u.z; r[3] += kc * u.w;
        __builtin_nontemporal_store(r, reinterpret_cast<floatx4 *>(S + size_t(c) * DV) + cg);
    }
    if (rg == 0) {
        const float kq = skq;
        store4(o + ch * DV + 4 * cg, Y.x + kq * u.x, Y.y + kq * u.y, Y.z + kq * u.z, Y.w + kq * u.w);
    }
}

template <class T, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int NH, hipStream_t s) {
    if (NH == 0) return hipSuccess;
    prof_begin(s);
    hipLaunchKernelGGL((kda_decode_kernel<T, DK, DV>), dim3(NH), dim3(256), 0, s,
                       static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), g, beta,
                       state, static_cast<T *>(o));
    prof_end(s, "kda_decode");
    return hipGetLastError();
}

template <class T>
static hipError_t decode_dispatch(int dk, int dv, const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int NH, hipStream_t s) {
#define KDA_DEC(DK_, DV_) \
    if (dk == DK_ && dv == DV_) return launch_decode_t<T, DK_, DV_>(q, k, v, g, beta, state, o, NH, s);
    KDA_DEC(32, 32) KDA_DEC(32, 64) KDA_DEC(32, 128)
    KDA_DEC(64, 32) KDA_DEC(64, 64) KDA_DEC(64, 128)
    KDA_DEC(128, 32) KDA_DEC(128, 64) KDA_DEC(128, 128)
#undef KDA_DEC
    return hipErrorInvalidValue;
}

hipError_t launch_decode(int dtype, const void *q, const void *k, const void *v, const float *g,
                         const float *beta, float *state, void *o, int N, int H, int dk, int dv,
                         hipStream_t s) {
    const int NH = N * H;
    if (dtype == 1) return decode_dispatch<bf16>(dk, dv, q, k, v, g, beta, state, o, NH, s);
    return decode_dispatch<float>(dk, dv, q, k, v, g, beta, state, o, NH, s);
}

}  // namespace kda
