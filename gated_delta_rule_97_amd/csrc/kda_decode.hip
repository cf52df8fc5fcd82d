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

// Threads per workgroup of the single-token step: each thread holds a 4 x 4
// block of the state (4 rows, one float4 of columns).  Small per-thread
// slices keep the register count low enough for eight waves per SIMD, so
// many (sequence, head) states are streaming at once on every compute unit.
template <int DK, int DV>
constexpr int decode_threads() {
    constexpr int n = (DV / 4) * DK / 4;
    return n < 64 ? 64 : (n > 1024 ? 1024 : n);
}

template <class T, int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void kda_decode_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                        const T *__restrict__ v, const float *__restrict__ g,
                                                        const float *__restrict__ beta, float *__restrict__ state,
                                                        T *__restrict__ o) {
    constexpr int CG = DV / 4;      // float4 column groups
    constexpr int RG = NTH / CG;    // row groups
    constexpr int RPT = DK / RG;    // rows per thread
    constexpr int NW = NTH / kWave; // wavefronts
    static_assert(RG * CG == NTH && RPT * RG == DK && RPT >= 1, "decode thread split");
    static_assert(CG <= kWave && kWave % CG == 0, "a wave spans whole row groups");
    __shared__ float sk[DK], sq[DK], sd[DK];
    __shared__ float4 sw[NW][CG], sy[NW][CG];
    __shared__ float skq;

    const size_t ch = blockIdx.x;  // sequence * H + head
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int lane = tid & (kWave - 1), wid = tid / kWave;
    float *S = state + ch * DK * DV;

    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)  // rows i*RG + rg: a workgroup-wide load is one contiguous span
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);
    for (int c = tid; c < DK; c += NTH) {
        sk[c] = to_f32(k[ch * DK + c]);
        sq[c] = to_f32(q[ch * DK + c]);
        sd[c] = exp_e(g[ch * DK + c]);
    }
    __syncthreads();
    if (tid < kWave) {
        float p = 0.f;
        for (int c = tid; c < DK; c += kWave) p += sk[c] * sq[c];
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) p += __shfl_xor(p, off);
        if (tid == 0) skq = p;
    }
    // partial w = S'^T k and y = S'^T q over this thread's rows, then over
    // the row groups of the wave (lanes CG apart), then over the waves
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f), y = w;
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
        const int c = i * RG + rg;
        const float f = sd[c], kc = sk[c], qc = sq[c];
        s[i] *= f;
        w.x += kc * s[i][0]; w.y += kc * s[i][1]; w.z += kc * s[i][2]; w.w += kc * s[i][3];
        y.x += qc * s[i][0]; y.y += qc * s[i][1]; y.z += qc * s[i][2]; y.w += qc * s[i][3];
    }
#pragma unroll
    for (int off = CG; off < kWave; off <<= 1) {
        w.x += __shfl_xor(w.x, off); w.y += __shfl_xor(w.y, off);
        w.z += __shfl_xor(w.z, off); w.w += __shfl_xor(w.w, off);
        y.x += __shfl_xor(y.x, off); y.y += __shfl_xor(y.y, off);
        y.z += __shfl_xor(y.z, off); y.w += __shfl_xor(y.w, off);
    }
    if (lane < CG) {
        sw[wid][cg] = w;
        sy[wid][cg] = y;
    }
    __syncthreads();
    float4 W = make_float4(0.f, 0.f, 0.f, 0.f), Y = W;
#pragma unroll
    for (int r = 0; r < NW; ++r) {
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

// ---------------------------------------------------------------------------
// Several decode tokens per sequence with the state held in registers
// (speculative decoding, serving-stack section of the blog post: drafted
// tokens are checked against the committed state, then the accepted ones
// are committed).  Inputs are [N][K][H][d] (token t of sequence n at row
// n * K + t).  VERIFY: all K tokens, o written per token, the state only
// read.  COMMIT: the first n_accept[n] (clamped to [0, K]) tokens of
// sequence n, no o, the state written back once (not at all when zero
// tokens are accepted).  Same per-token arithmetic as kda_decode_kernel.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int CPB, bool VERIFY>
__global__ __launch_bounds__(256) void kda_decode_multi_kernel(const T *__restrict__ q, const T *__restrict__ k,
                                                                 const T *__restrict__ v, const float *__restrict__ g,
                                                                 const float *__restrict__ beta,
                                                                 const int32_t *__restrict__ n_accept,
                                                                 float *__restrict__ state, T *__restrict__ o, int K,
                                                                 int H) {
    constexpr int CG = CPB / 4;   // float4 column groups of this workgroup's CPB value columns
    constexpr int RG = 256 / CG;
    constexpr int RPT = DK / RG;
    constexpr int KG = 8;  // draft tokens staged in LDS at once
    static_assert(DV % CPB == 0, "column blocks");
    static_assert(RG * CG == 256 && RPT * RG == DK, "decode thread split");
    // a group's k, q and e^g, and the row-group partials of two tokens in turn
    __shared__ float sk[KG][DK], sq[VERIFY ? KG : 1][DK], sd[KG][DK];
    __shared__ float4 sw[2][RG][CG], sy[VERIFY ? 2 : 1][RG][CG];
    __shared__ float skq[KG];

    // the value columns of S are independent: (sequence, head) spans DV / CPB
    // workgroups, each the state's columns cb * CPB ..
    const int ch = blockIdx.x / (DV / CPB), cb = blockIdx.x % (DV / CPB);  // ch = sequence * H + head
    const int n = ch / H, h = ch - n * H;
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    const int col0 = cb * CPB;
    int ntok = K;
    if (!VERIFY) {
        const int na = n_accept[n];
        ntok = na < 0 ? 0 : (na > K ? K : na);
        if (ntok == 0) return;  // nothing accepted: the state stays as it is
    }
    float *S = state + size_t(ch) * DK * DV + col0;

    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);

    for (int t0 = 0; t0 < ntok; t0 += KG) {
        const int nt = min(KG, ntok - t0);
        __syncthreads();  // the previous group's last reads of sk/sq/sd are done
        for (int i = tid; i < nt * DK; i += 256) {
            const int t = i / DK, c = i - t * DK;
            const size_t row = (size_t(n) * K + t0 + t) * H + h;  // token row of [N][K][H]
            sk[t][c] = to_f32(k[row * DK + c]);
            if (VERIFY) sq[t][c] = to_f32(q[row * DK + c]);
            sd[t][c] = exp_e(g[row * DK + c]);
        }
        __syncthreads();
        if (VERIFY) {  // k . q of each token: one wave per token
            for (int t = tid >> 6; t < nt; t += 4) {
                float p = 0.f;
                for (int c = tid & 63; c < DK; c += 64) p += sk[t][c] * sq[t][c];
#pragma unroll
                for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
                if ((tid & 63) == 0) skq[t] = p;
            }
        }
        for (int t = 0; t < nt; ++t) {
            const int pb = t & 1;
            float4 w = make_float4(0.f, 0.f, 0.f, 0.f), y = w;
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int c = i * RG + rg;
                const float f = sd[t][c], kc = sk[t][c];
                s[i] *= f;
                w.x += kc * s[i][0]; w.y += kc * s[i][1]; w.z += kc * s[i][2]; w.w += kc * s[i][3];
                if (VERIFY) {
                    const float qc = sq[t][c];
                    y.x += qc * s[i][0]; y.y += qc * s[i][1]; y.z += qc * s[i][2]; y.w += qc * s[i][3];
                }
            }
            sw[pb][rg][cg] = w;
            if (VERIFY) sy[pb][rg][cg] = y;
            __syncthreads();  // one barrier per token: the partials of two tokens alternate
            float4 W = make_float4(0.f, 0.f, 0.f, 0.f), Y = W;
#pragma unroll
            for (int r = 0; r < RG; ++r) {
                const float4 a4 = sw[pb][r][cg];
                W.x += a4.x; W.y += a4.y; W.z += a4.z; W.w += a4.w;
                if (VERIFY) {
                    const float4 b4 = sy[pb][r][cg];
                    Y.x += b4.x; Y.y += b4.y; Y.z += b4.z; Y.w += b4.w;
                }
            }
            const size_t row = (size_t(n) * K + t0 + t) * H + h;
            const float bt = beta[row];
            const T *vp = v + row * DV + col0 + 4 * cg;
            float4 u;
            u.x = bt * (to_f32(vp[0]) - W.x);
            u.y = bt * (to_f32(vp[1]) - W.y);
            u.z = bt * (to_f32(vp[2]) - W.z);
            u.w = bt * (to_f32(vp[3]) - W.w);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float kc = sk[t][i * RG + rg];
                s[i][0] += kc * u.x; s[i][1] += kc * u.y; s[i][2] += kc * u.z; s[i][3] += kc * u.w;
            }
            if (VERIFY && rg == 0) {
                const float kq = skq[t];
                store4(o + row * DV + col0 + 4 * cg, Y.x + kq * u.x, Y.y + kq * u.y, Y.z + kq * u.z,
                       Y.w + kq * u.w);
            }
        }
    }
    if (!VERIFY) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);
    }
}

template <class T, int DK, int DV, bool VERIFY>
static hipError_t launch_multi_t(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                 const int32_t *n_accept, float *state, void *o, int N, int K, int H,
                                 hipStream_t s) {
    if (N == 0 || K == 0) return hipSuccess;
    // all value columns in one workgroup: splitting them repeats the token
    // staging and doubles the row-group partials each reduction reads (slower)
    constexpr int CPB = DV;
    prof_begin(s);
    hipLaunchKernelGGL((kda_decode_multi_kernel<T, DK, DV, CPB, VERIFY>), dim3(N * H * (DV / CPB)), dim3(256), 0, s,
                       static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), g, beta,
                       n_accept, state, static_cast<T *>(o), K, H);
    prof_end(s, VERIFY ? "kda_decode_verify" : "kda_decode_commit");
    return hipGetLastError();
}

template <class T, bool VERIFY>
static hipError_t multi_dispatch(int dk, int dv, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const int32_t *n_accept, float *state, void *o, int N, int K,
                                 int H, hipStream_t s) {
#define KDA_MUL(DK_, DV_) \
    if (dk == DK_ && dv == DV_) \
        return launch_multi_t<T, DK_, DV_, VERIFY>(q, k, v, g, beta, n_accept, state, o, N, K, H, s);
    KDA_MUL(32, 32) KDA_MUL(32, 64) KDA_MUL(32, 128)
    KDA_MUL(64, 32) KDA_MUL(64, 64) KDA_MUL(64, 128)
    KDA_MUL(128, 32) KDA_MUL(128, 64) KDA_MUL(128, 128)
#undef KDA_MUL
    return hipErrorInvalidValue;
}

hipError_t launch_decode_verify(int dtype, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *state, void *o, int N, int K, int H, int dk,
                                int dv, hipStream_t s) {
    float *st = const_cast<float *>(state);  // read only in this mode
    if (dtype == 1) return multi_dispatch<bf16, true>(dk, dv, q, k, v, g, beta, nullptr, st, o, N, K, H, s);
    return multi_dispatch<float, true>(dk, dv, q, k, v, g, beta, nullptr, st, o, N, K, H, s);
}

hipError_t launch_decode_commit(int dtype, const void *k, const void *v, const float *g, const float *beta,
                                const int32_t *n_accept, float *state, int N, int K, int H, int dk, int dv,
                                hipStream_t s) {
    if (dtype == 1) return multi_dispatch<bf16, false>(dk, dv, nullptr, k, v, g, beta, n_accept, state, nullptr, N,
                                                       K, H, s);
    return multi_dispatch<float, false>(dk, dv, nullptr, k, v, g, beta, n_accept, state, nullptr, N, K, H, s);
}

template <class T, int DK, int DV>
static hipError_t launch_decode_t(const void *q, const void *k, const void *v, const float *g,
                                  const float *beta, float *state, void *o, int NH, hipStream_t s) {
    if (NH == 0) return hipSuccess;
    constexpr int NTH = decode_threads<DK, DV>();
    prof_begin(s);
    hipLaunchKernelGGL((kda_decode_kernel<T, DK, DV, NTH>), dim3(NH), dim3(NTH), 0, s,
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
