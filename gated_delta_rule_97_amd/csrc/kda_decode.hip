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
#include <type_traits>

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// Cross-lane moves on the VALU (no LDS traffic): xor 8 stays inside a
// 16-lane row (DPP row_ror:8); v_permlane16_swap exchanges the odd 16-lane
// rows of its first operand with the even rows of its second, so (x, y)
// becomes (x_r0 | y_r0 | x_r2 | y_r2, x_r1 | y_r1 | x_r3 | y_r3); and
// v_permlane32_swap exchanges the upper 32 lanes of its first operand with
// the lower 32 lanes of its second: (x, y) becomes (x_lo | y_lo, x_hi | y_hi).
__device__ __forceinline__ float lane_xor8(float x) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ void lane_swap16(float x, float y, float &xs, float &ys) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    xs = __uint_as_float(r[0]);
    ys = __uint_as_float(r[1]);
}
__device__ __forceinline__ void lane_swap32(float x, float y, float &xs, float &ys) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
    xs = __uint_as_float(r[0]);
    ys = __uint_as_float(r[1]);
}

// Sum over all 64 lanes, in every lane: the halves and the row pairs by
// swaps, then rotations inside each 16-lane row.
__device__ __forceinline__ float wave_sum(float x) {
    float a, b;
    lane_swap32(x, x, a, b);
    x = a + b;
    lane_swap16(x, x, a, b);
    x = a + b;
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x128, 0xF, 0xF, false));  // row_ror:8
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x124, 0xF, 0xF, false));  // row_ror:4
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x122, 0xF, 0xF, false));  // row_ror:2
    x += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x121, 0xF, 0xF, false));  // row_ror:1
    return x;
}

// For a wave whose lanes are 8 * row group + column group: the sum of a
// float4 over the eight row groups, reduce-scattered: the lanes
// whose row-group bits 4 and 5 are b4 and b5 get the sum of component
// 2 b5 + b4 (both lanes of a bit-3 pair the same value).  Each halving
// moves only the components the partner keeps.
__device__ __forceinline__ float rg_sum_scatter(floatx4 x, int b4, int b5) {
    float p0, p1, q0, q1;
    lane_swap32(x[0], x[2], p0, p1);  // p0 + p1: component 0 in the lower half, 2 in the upper
    lane_swap32(x[1], x[3], q0, q1);
    const float a = p0 + p1, b = q0 + q1;  // components 2 b5 and 2 b5 + 1
    float a2, b2;
    lane_swap16(a, b, a2, b2);
    const float r = a2 + b2;  // component 2 b5 in even rows, 2 b5 + 1 in odd rows
    return r + lane_xor8(r);
}

// The inverse gather: lane (b4, b5) holds component 2 b5 + b4; every lane
// gets all four.
__device__ __forceinline__ floatx4 rg_gather(float x, int b4, int b5) {
    float xe, xo;
    lane_swap16(x, x, xe, xo);  // xe: even rows' values in each row pair, xo: odd rows'
    const float o = b4 ? xe : xo;  // component 2 b5 + 1 - b4
    const float lo = b4 ? o : x, hi = b4 ? x : o;  // components 2 b5, 2 b5 + 1
    float p0, p1, q0, q1;
    lane_swap32(lo, hi, p0, p1);  // lower half: p1 = component 2; upper half: p0 = component 1
    lane_swap32(hi, lo, q0, q1);  // lower half: q1 = component 3; upper half: q0 = component 0
    return b5 ? floatx4{q0, p0, lo, hi} : floatx4{lo, hi, p1, q1};
}

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
    static_assert(CG <= kWave / 2, "row group 0 lies in wave 0");
    __shared__ float sk[DK], sq[DK], sd[DK];
    __shared__ float4 sw[NW][CG], sy[NW][CG];

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
    if constexpr (2 * CG == kWave) {
        // the wave's two row groups are its 32-lane halves: one swap per
        // component leaves w's sums in the lower half and y's in the upper
        float4 r;
        float p, q;
        lane_swap32(w.x, y.x, p, q); r.x = p + q;
        lane_swap32(w.y, y.y, p, q); r.y = p + q;
        lane_swap32(w.z, y.z, p, q); r.z = p + q;
        lane_swap32(w.w, y.w, p, q); r.w = p + q;
        if (lane < CG) sw[wid][cg] = r;
        else sy[wid][cg] = r;
    } else {
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
    if (wid == 0) {  // the o row: row group 0 lies in wave 0, which also sums k . q
        float kq = 0.f;
        for (int c = lane; c < DK; c += kWave) kq += sk[c] * sq[c];
        kq = wave_sum(kq);
        if (rg == 0) store4(o + ch * DV + 4 * cg, Y.x + kq * u.x, Y.y + kq * u.y, Y.z + kq * u.z, Y.w + kq * u.w);
    }
}

// ---------------------------------------------------------------------------
// Several decode tokens per sequence with the state held in registers
// (speculative decoding, serving-stack section of the blog post: drafted
// tokens are checked against the committed state, then the accepted ones
// are committed).  Inputs are [N][K][H][d] (token t of sequence n at row
// n * K + t).  kVerify: all K tokens, o written per token, the state only
// read.  kCommit: the first n_accept[n] (clamped to [0, K]) tokens of
// sequence n, no o, the state written back once (not at all when zero
// tokens are accepted).  kStep: one token, o and the state (a decode step).
//
// Every value column of the state evolves on its own: w = S'^T k, u, the
// update k u^T and o = S^T q are all per column, and only k, q, e^g and beta
// are shared.  So one wavefront holds CW value columns x all DK rows of one
// (sequence, head) and needs no other wave: each lane owns RPT consecutive
// rows of one float4 of columns, and the reductions over dk sum a lane's
// rows and then its row groups by cross-lane moves.  No barrier.
// ---------------------------------------------------------------------------
enum DecodeMode { kVerify = 0, kCommit = 1, kStep = 2, kCommitVerify = 3 };

template <int DV>
constexpr int wave_columns() { return DV < 32 ? DV : 32; }

// Per-token vectors of a group of KG tokens are staged once per wave in the
// wave's own LDS region (one 16-byte unit per lane and load, e^g taken once
// per element) and each lane reads its rows from there: read by every lane
// straight from memory they would cost one load per 16-byte unit per lane,
// and eight lanes share each row group.  The region belongs to one wave, and
// a wave's LDS accesses complete in order, so no workgroup barrier is needed;
// wave_lds_sync() marks each point where lanes start reading what other lanes
// wrote, or overwrite what other lanes read, so that the compiler keeps every
// LDS access on its side of that point.
constexpr int kWaveKG = 4;   // tokens staged at once
constexpr int kWavePB = 4;   // waves per workgroup

template <int DK>
__device__ __forceinline__ int wave_vec_idx(int c) { return c + (c >> 4) * 4; }  // 4-float pad per 16: row groups hit distinct banks

template <class T, int DK, int DV, int MODE>
__global__ __launch_bounds__(kWavePB * kWave, 4) void kda_decode_wave_kernel(
    const T *__restrict__ q, const T *__restrict__ k, const T *__restrict__ v, const float *__restrict__ g,
    const float *__restrict__ beta, const int32_t *__restrict__ n_accept, float *__restrict__ state,
    T *__restrict__ o, float *__restrict__ u_out, int K, int H, int nwaves, const T *__restrict__ pk,
    const float *__restrict__ pg, const float *__restrict__ pu, const int32_t *__restrict__ pacc, int Kp) {
    constexpr int CW = wave_columns<DV>();  // value columns of one wave
    constexpr int CG = CW / 4;              // float4 column groups: lanes cg = lane % CG
    constexpr int RG = kWave / CG;          // row groups: lanes rg = lane / CG
    constexpr int RPT = DK / RG;            // consecutive rows per lane
    constexpr int NB = DV / CW;             // waves per (sequence, head)
    constexpr bool OUT = MODE != kCommit, WRITE = MODE == kCommit || MODE == kStep;
    static_assert(CG * RG == kWave && RPT * RG == DK && RPT % 4 == 0 && DV % CW == 0, "decode wave split");
    static_assert(CG == 8, "row groups are lane bits 3..5");
    constexpr int NVEC = OUT ? 3 : 2;                   // staged per token: k, e^g (, q), as fp32
    constexpr int DKP = DK + DK / 4;                    // padded row of one vector
    constexpr int EPU = 16 / int(sizeof(T));            // values of T per 16-byte unit
    constexpr int KU = DK / EPU, GU = DK / 4;           // 16-byte units of k (and q), of g
    __shared__ __align__(16) float sv[kWavePB][kWaveKG][NVEC][DKP];

    const int wv = blockIdx.x * kWavePB + int(threadIdx.x / kWave);
    if (wv >= nwaves) return;  // no barrier anywhere: a wave past the end simply leaves
    const int ch = wv / NB, cb = wv - ch * NB;  // ch = sequence * H + head
    const int n = ch / H, h = ch - n * H;
    const int lane = threadIdx.x & (kWave - 1), cg = lane % CG, rg = lane / CG;
    const int r0 = rg * RPT, col = cb * CW + 4 * cg;
    const int b4 = (lane >> 4) & 1, b5 = lane >> 5, cj = 2 * b5 + b4;  // row-group bits 4, 5
    float(*my)[NVEC][DKP] = sv[threadIdx.x / kWave];
    int ntok = K;
    if (MODE == kCommit) {
        const int na = n_accept[n];
        ntok = na < 0 ? 0 : (na > K ? K : na);
        if (ntok == 0) return;  // nothing accepted: the state stays as it is
    }
    float *S = state + size_t(ch) * DK * DV + col;

    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + size_t(r0 + i) * DV));

    // Stage k, e^g (and q, for WQ) of tokens t0 .. t0 + nt - 1 of an [N][Kx][H]
    // input into the wave's LDS region (k in vector 0, e^g in 1, q in 2):
    // unit j of token tt, one 16-byte unit per lane and load
    auto stage = [&](auto wq, const T *kp, const T *qp, const float *gp, int Kx, int t0, int nt) {
        constexpr bool WQ = decltype(wq)::value;
        constexpr int UTx = KU * (WQ ? 2 : 1) + GU;  // units per token
        constexpr int ITx = (kWaveKG * UTx + kWave - 1) / kWave;
        u32x4 raw[ITx];
#pragma unroll
        for (int it = 0; it < ITx; ++it) {
            const int u = min(lane + kWave * it, nt * UTx - 1);  // past the group: a repeated (unused) load
            const int tt = u / UTx, j = u - tt * UTx;
            const size_t row = (size_t(n) * Kx + t0 + tt) * H + h;
            const char *src = (j < KU) ? reinterpret_cast<const char *>(kp + row * DK) + 16 * j
                              : (WQ && j < 2 * KU) ? reinterpret_cast<const char *>(qp + row * DK) + 16 * (j - KU)
                                                   : reinterpret_cast<const char *>(gp + row * DK) +
                                                         16 * (j - (WQ ? 2 : 1) * KU);
            raw[it] = *reinterpret_cast<const u32x4 *>(src);
        }
        wave_lds_sync();  // the previous group's reads of the region are behind
#pragma unroll
        for (int it = 0; it < ITx; ++it) {
            const int u = lane + kWave * it;
            if (u < nt * UTx) {
                const int tt = u / UTx, j = u - tt * UTx;
                if (j < (WQ ? 2 : 1) * KU) {  // k or q: EPU values of T
                    const int vi = j < KU ? 0 : 2, c0 = EPU * (j < KU ? j : j - KU);
                    float *d = &my[tt][vi][wave_vec_idx<DK>(c0)];
                    if constexpr (sizeof(T) == 2) {
                        float f[8];
#pragma unroll
                        for (int e2 = 0; e2 < 4; ++e2) {
                            f[2 * e2] = __uint_as_float(raw[it][e2] << 16);
                            f[2 * e2 + 1] = __uint_as_float(raw[it][e2] & 0xffff0000u);
                        }
                        *reinterpret_cast<floatx4 *>(d) = floatx4{f[0], f[1], f[2], f[3]};
                        *reinterpret_cast<floatx4 *>(d + 4) = floatx4{f[4], f[5], f[6], f[7]};
                    } else {
                        *reinterpret_cast<u32x4 *>(d) = raw[it];
                    }
                } else {  // g: four values, stored as e^g
                    const int c0 = 4 * (j - (WQ ? 2 : 1) * KU);
                    *reinterpret_cast<floatx4 *>(&my[tt][1][wave_vec_idx<DK>(c0)]) =
                        floatx4{exp_e(__uint_as_float(raw[it][0])), exp_e(__uint_as_float(raw[it][1])),
                                exp_e(__uint_as_float(raw[it][2])), exp_e(__uint_as_float(raw[it][3]))};
                }
            }
        }
        wave_lds_sync();  // the group is staged
    };

    if constexpr (MODE == kCommitVerify) {
        // the previous round's accepted drafts first, from the update vectors
        // its verify kept: per token S' = Diag(e^g) S, then S = S' + k u^T, the
        // commit's own two steps with u known (no reduction over dk); the
        // committed state is written once, then verified from
        const int pa = pacc ? pacc[n] : 0;
        const int np = pa < 0 ? 0 : (pa > Kp ? Kp : pa);
        static_assert(NVEC == 3 && CW <= DKP, "the q slot of the staging region holds u");
        for (int t0 = 0; t0 < np; t0 += kWaveKG) {
            const int nt = min(kWaveKG, np - t0);
            wave_lds_sync();  // the previous group's reads of u are behind
            // u of the wave's CW columns, staged in the (here unused) q slot
            if (lane < CG * nt) {
                const int tt = lane / CG, c4 = lane - tt * CG;
                const size_t prow = (size_t(n) * Kp + t0 + tt) * H + h;
                *reinterpret_cast<floatx4 *>(&my[tt][2][4 * c4]) =
                    *reinterpret_cast<const floatx4 *>(pu + prow * DV + cb * CW + 4 * c4);
            }
            stage(std::integral_constant<bool, false>{}, pk, nullptr, pg, Kp, t0, nt);
            for (int tt = 0; tt < nt; ++tt) {
                const float *kv = &my[tt][0][wave_vec_idx<DK>(r0)];
                const float *ev = &my[tt][1][wave_vec_idx<DK>(r0)];
                const floatx4 ut = *reinterpret_cast<const floatx4 *>(&my[tt][2][4 * cg]);
#pragma unroll
                for (int i = 0; i < RPT; i += 4) {
                    const floatx4 k4 = *reinterpret_cast<const floatx4 *>(kv + i);
                    const floatx4 e4 = *reinterpret_cast<const floatx4 *>(ev + i);
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        s[i + j] *= e4[j];
                        s[i + j] += k4[j] * ut;
                    }
                }
            }
        }
        if (np > 0) {
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4 *>(S + size_t(r0 + i) * DV));
        }
    }

    for (int t0 = 0; t0 < ntok; t0 += kWaveKG) {
        const int nt = min(kWaveKG, ntok - t0);
        stage(std::integral_constant<bool, OUT>{}, k, q, g, K, t0, nt);
        // ---- the group's tokens, one after the other ----
        for (int tt = 0; tt < nt; ++tt) {
            const size_t row = (size_t(n) * K + t0 + tt) * H + h;  // token row of [N][K][H]
            const float *kv = &my[tt][0][wave_vec_idx<DK>(r0)];
            const float *ev = &my[tt][1][wave_vec_idx<DK>(r0)];
            float kf[RPT];
            floatx4 w = zero4();
#pragma unroll
            for (int i = 0; i < RPT; i += 4) {
                const floatx4 k4 = *reinterpret_cast<const floatx4 *>(kv + i);
                const floatx4 e4 = *reinterpret_cast<const floatx4 *>(ev + i);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    kf[i + j] = k4[j];
                    s[i + j] *= e4[j];  // decay, then the partial sum of w = S'^T k
                    w += k4[j] * s[i + j];
                }
            }
            // lane (b4, b5) finishes column cj of its group: w, then u = beta (v - w)
            const float wj = rg_sum_scatter(w, b4, b5);
            const float uj = beta[row] * (to_f32(v[row * DV + col + cj]) - wj);
            const floatx4 u = rg_gather(uj, b4, b5);
#pragma unroll
            for (int i = 0; i < RPT; ++i) s[i] += kf[i] * u;
            if constexpr (MODE == kVerify || MODE == kCommitVerify)  // kept for a commit from it
                if (u_out && !(lane & CG)) u_out[row * DV + col + cj] = uj;
            if constexpr (OUT) {  // o = S^T q of the updated state
                const float *qv = &my[tt][2][wave_vec_idx<DK>(r0)];
                floatx4 y = zero4();
#pragma unroll
                for (int i = 0; i < RPT; i += 4) {
                    const floatx4 q4 = *reinterpret_cast<const floatx4 *>(qv + i);
#pragma unroll
                    for (int j = 0; j < 4; ++j) y += q4[j] * s[i + j];
                }
                const float yj = rg_sum_scatter(y, b4, b5);
                if (!(lane & CG)) o[row * DV + col + cj] = from_f32<T>(yj);
            }
        }
    }
    if constexpr (WRITE) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4 *>(S + size_t(r0 + i) * DV));
    }
}

struct PrevRound {  // the previous round's drafts, for a commit in front of a verify
    const void *k = nullptr;
    const float *g = nullptr, *u = nullptr;
    const int32_t *n_accept = nullptr;
    int K = 0;
};

template <class T, int DK, int DV, int MODE>
static hipError_t launch_wave_t(const void *q, const void *k, const void *v, const float *g, const float *beta,
                                const int32_t *n_accept, float *state, void *o, float *u_out, int N, int K, int H,
                                hipStream_t s, const char *name, const PrevRound &pr = PrevRound{}) {
    if (N == 0 || K == 0) return hipSuccess;
    constexpr int NB = DV / wave_columns<DV>();
    const int nwaves = N * H * NB;
    constexpr int WPB = kWavePB;  // the column blocks of one (sequence, head) share a CU at DV = 128
    prof_begin(s);
    hipLaunchKernelGGL((kda_decode_wave_kernel<T, DK, DV, MODE>), dim3((nwaves + WPB - 1) / WPB), dim3(WPB * kWave),
                       0, s, static_cast<const T *>(q), static_cast<const T *>(k), static_cast<const T *>(v), g, beta,
                       n_accept, state, static_cast<T *>(o), u_out, K, H, nwaves, static_cast<const T *>(pr.k), pr.g,
                       pr.u, pr.n_accept, pr.K);
    prof_end(s, name);
    return hipGetLastError();
}

template <class T, bool VERIFY>
static hipError_t multi_dispatch(int dk, int dv, const void *q, const void *k, const void *v, const float *g,
                                 const float *beta, const int32_t *n_accept, float *state, void *o, float *u_out,
                                 int N, int K, int H, hipStream_t s) {
#define KDA_MUL(DK_, DV_)                                                                                          \
    if (dk == DK_ && dv == DV_)                                                                                    \
        return VERIFY ? launch_wave_t<T, DK_, DV_, kVerify>(q, k, v, g, beta, n_accept, state, o, u_out, N, K, H, \
                                                            s, "kda_decode_verify")                                \
                      : launch_wave_t<T, DK_, DV_, kCommit>(q, k, v, g, beta, n_accept, state, o, nullptr, N, K,   \
                                                            H, s, "kda_decode_commit");
    KDA_MUL(32, 32) KDA_MUL(32, 64) KDA_MUL(32, 128)
    KDA_MUL(64, 32) KDA_MUL(64, 64) KDA_MUL(64, 128)
    KDA_MUL(128, 32) KDA_MUL(128, 64) KDA_MUL(128, 128)
#undef KDA_MUL
    return hipErrorInvalidValue;
}

hipError_t launch_decode_verify(int dtype, const void *q, const void *k, const void *v, const float *g,
                                const float *beta, const float *state, void *o, float *u_out, int N, int K, int H,
                                int dk, int dv, hipStream_t s) {
    float *st = const_cast<float *>(state);  // read only in this mode
    if (dtype == 1) return multi_dispatch<bf16, true>(dk, dv, q, k, v, g, beta, nullptr, st, o, u_out, N, K, H, s);
    return multi_dispatch<float, true>(dk, dv, q, k, v, g, beta, nullptr, st, o, u_out, N, K, H, s);
}

template <class T>
static hipError_t commit_verify_dispatch(int dk, int dv, const void *q, const void *k, const void *v,
                                         const float *g, const float *beta, float *state, void *o, float *u_out,
                                         int N, int K, int H, const PrevRound &pr, hipStream_t s) {
#define KDA_CV(DK_, DV_)                                                                                          \
    if (dk == DK_ && dv == DV_)                                                                                   \
        return launch_wave_t<T, DK_, DV_, kCommitVerify>(q, k, v, g, beta, nullptr, state, o, u_out, N, K, H, s,  \
                                                         "kda_decode_commit_verify", pr);
    KDA_CV(32, 32) KDA_CV(32, 64) KDA_CV(32, 128)
    KDA_CV(64, 32) KDA_CV(64, 64) KDA_CV(64, 128)
    KDA_CV(128, 32) KDA_CV(128, 64) KDA_CV(128, 128)
#undef KDA_CV
    return hipErrorInvalidValue;
}

hipError_t launch_decode_commit_verify(int dtype, const void *pk, const float *pg, const float *pu,
                                       const int32_t *pacc, int Kp, const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, float *state, void *o, float *u_out,
                                       int N, int K, int H, int dk, int dv, hipStream_t s) {
    PrevRound pr;
    pr.k = pk; pr.g = pg; pr.u = pu; pr.n_accept = pacc; pr.K = Kp;
    if (dtype == 1) return commit_verify_dispatch<bf16>(dk, dv, q, k, v, g, beta, state, o, u_out, N, K, H, pr, s);
    return commit_verify_dispatch<float>(dk, dv, q, k, v, g, beta, state, o, u_out, N, K, H, pr, s);
}

hipError_t launch_decode_commit(int dtype, const void *k, const void *v, const float *g, const float *beta,
                                const int32_t *n_accept, float *state, int N, int K, int H, int dk, int dv,
                                hipStream_t s) {
    if (dtype == 1) return multi_dispatch<bf16, false>(dk, dv, nullptr, k, v, g, beta, n_accept, state, nullptr,
                                                       nullptr, N, K, H, s);
    return multi_dispatch<float, false>(dk, dv, nullptr, k, v, g, beta, n_accept, state, nullptr, nullptr, N, K, H,
                                        s);
}

// Commit from the update vectors a verify kept (same committed state, same
// drafts).  Unrolling the recurrence S_t = Diag(e^{g_t}) S_{t-1} + k_t u_t^T
// over the first n drafts gives
//   S_n = Diag(D_0) S_0 + sum_{t<n} Diag(D_{t+1}) k_t u_t^T,
// where D_t is the per-row product of e^g over drafts t .. n-1 (D_n = 1), so
// with u_t known no reduction over dk is left: per group of up to KG drafts
// the factors D_{t+1} k_t and D_0 of each row are formed in LDS, and every
// thread updates its 4 x 4 blocks (the single-step layout) with one multiply
// and one FMA per draft.  The state is read and written once.
template <class T, int DK, int DV, int NTH>
__global__ __launch_bounds__(NTH) void kda_decode_commit_kept_kernel(const T *__restrict__ k,
                                                                     const float *__restrict__ g,
                                                                     const float *__restrict__ u,
                                                                     const int32_t *__restrict__ n_accept,
                                                                     float *__restrict__ state, int K, int H) {
    constexpr int CG = DV / 4;    // float4 column groups
    constexpr int RG = NTH / CG;  // row groups
    constexpr int RPT = DK / RG;  // rows per thread
    constexpr int KG = 8;         // drafts per staged group
    static_assert(RG * CG == NTH && RPT * RG == DK && RPT >= 1, "commit thread split");
    __shared__ float sk[KG][DK], se[KG][DK], sf[KG][DK], sd[DK];
    __shared__ floatx4 su[KG][CG];

    const int ch = blockIdx.x;  // sequence * H + head
    const int n = ch / H, h = ch - n * H;
    const int na0 = n_accept[n];
    const int na = na0 < 0 ? 0 : (na0 > K ? K : na0);
    if (na == 0) return;  // the whole workgroup leaves: nothing accepted
    const int tid = threadIdx.x, cg = tid % CG, rg = tid / CG;
    float *S = state + size_t(ch) * DK * DV;
    floatx4 s[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i)  // rows i * RG + rg
        s[i] = __builtin_nontemporal_load(reinterpret_cast<const floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);
    for (int g0 = 0; g0 < na; g0 += KG) {
        const int ng = min(KG, na - g0);
        if (g0 > 0) __syncthreads();  // the previous group's factors are read
        for (int e = tid; e < ng * DK; e += NTH) {
            const int t = e / DK, c = e - t * DK;
            const size_t row = (size_t(n) * K + g0 + t) * H + h;
            sk[t][c] = to_f32(k[row * DK + c]);
            se[t][c] = exp_e(g[row * DK + c]);
        }
        for (int e = tid; e < ng * CG; e += NTH) {
            const int t = e / CG, c4 = e - t * CG;
            su[t][c4] = reinterpret_cast<const floatx4 *>(u + ((size_t(n) * K + g0 + t) * H + h) * DV)[c4];
        }
        __syncthreads();
        for (int r = tid; r < DK; r += NTH) {
            float p = 1.f;
            for (int t = ng - 1; t >= 0; --t) {
                sf[t][r] = sk[t][r] * p;
                p *= se[t][r];
            }
            sd[r] = p;
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const int r = i * RG + rg;
            floatx4 acc = sd[r] * s[i];
            for (int t = 0; t < ng; ++t) acc += sf[t][r] * su[t][cg];
            s[i] = acc;
        }
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i)
        __builtin_nontemporal_store(s[i], reinterpret_cast<floatx4 *>(S + size_t(i * RG + rg) * DV) + cg);
}

template <class T, int DK, int DV>
static hipError_t launch_commit_kept_t(const void *k, const float *g, const float *u, const int32_t *n_accept,
                                       float *state, int N, int K, int H, hipStream_t s) {
    if (N == 0 || K == 0) return hipSuccess;
    constexpr int NTH = decode_threads<DK, DV>();
    prof_begin(s);
    hipLaunchKernelGGL((kda_decode_commit_kept_kernel<T, DK, DV, NTH>), dim3(N * H), dim3(NTH), 0, s,
                       static_cast<const T *>(k), g, u, n_accept, state, K, H);
    prof_end(s, "kda_decode_commit_kept");
    return hipGetLastError();
}

template <class T>
static hipError_t commit_kept_dispatch(int dk, int dv, const void *k, const float *g, const float *u,
                                       const int32_t *n_accept, float *state, int N, int K, int H, hipStream_t s) {
#define KDA_CK(DK_, DV_) \
    if (dk == DK_ && dv == DV_) return launch_commit_kept_t<T, DK_, DV_>(k, g, u, n_accept, state, N, K, H, s);
    KDA_CK(32, 32) KDA_CK(32, 64) KDA_CK(32, 128)
    KDA_CK(64, 32) KDA_CK(64, 64) KDA_CK(64, 128)
    KDA_CK(128, 32) KDA_CK(128, 64) KDA_CK(128, 128)
#undef KDA_CK
    return hipErrorInvalidValue;
}

hipError_t launch_decode_commit_kept(int dtype, const void *k, const float *g, const float *u,
                                     const int32_t *n_accept, float *state, int N, int K, int H, int dk, int dv,
                                     hipStream_t s) {
    if (dtype == 1) return commit_kept_dispatch<bf16>(dk, dv, k, g, u, n_accept, state, N, K, H, s);
    return commit_kept_dispatch<float>(dk, dv, k, g, u, n_accept, state, N, K, H, s);
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
