// Chunked KDA prefill kernels for gfx950.
//
// Method (Kimi K3 architecture blog post, section on the lower bound on the
// log-decay): the recurrent state is evaluated chunk by chunk; inside a chunk
// every pairwise decay exp(Gam_t - Gam_s) is a ratio of accumulated decays,
// i.e. a division by the accumulated decay.  Because every per-step
// log-decay is >= -5, a 16-token tile accumulates at least -80, so the
// reciprocal stays below e^80 (~5.5e34), inside bf16's range (~3.4e38): the
// diagonal tiles use the same dense MFMA as every other tile, with no
// pairwise special path.
//
// For one head, a chunk of C tokens entering with state S (dk x dv):
//   Gam_t = sum_{s<=t} g_s (per channel, from the chunk start)
//   r_I   = Gam just before 16-token tile I (0 for the first tile)
//   A_ts  = beta_t sum_c k_t[c] k_s[c] e^{Gam_t[c]-Gam_s[c]}      s < t
//   P_ts  = sum_c q_t[c] k_s[c] e^{Gam_t[c]-Gam_s[c]}             s <= t
//   tile pair (I, J<=I) factors the decay as
//     e^{Gam_t - r_I} (<= 1, row operand) * e^{r_I - Gam_s} (<= e^80, column)
//   L     = (I + A)^-1               blocked forward substitution, fp32
//   W     = L (beta k e^Gam),  Ut = L (beta v)                   (WY / UT form)
//   Q'    = q e^Gam - P W,     Oi = P Ut      (state-free part of the output)
// and, sequentially over chunks, with the state kept on chip in fp32:
//   U      = Ut - W S
//   o      = Oi + Q' S
//   S_next = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U
//
// Kernel 1 (kda_intra_kernel): one workgroup per (chunk, head), fully
//   parallel; everything that does not depend on the incoming state.
// Kernel 2 (kda_inter_kernel): one workgroup per (sequence, head, dv block),
//   sequential over the sequence's chunks; the fp32 state block lives in
//   MFMA accumulator registers for the whole sequence.
#pragma once

#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

constexpr int kThreads = 256;  // 4 wavefronts
constexpr int kWaves = kThreads / kWave;

// ---------------------------------------------------------------------------
// Where a chunk slot lives in the token stream.
// ---------------------------------------------------------------------------
struct ChunkLoc {
    int seq, tok0, len;
};

__device__ __forceinline__ int clampi(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ __forceinline__ bool locate_chunk(const PrefillArgs &a, int gc, int C, ChunkLoc &out) {
    if (!a.cu) {
        const int n = gc / a.nc_seq, ci = gc - n * a.nc_seq;
        if (n >= a.N) return false;
        out.seq = n;
        out.tok0 = n * a.T + ci * C;
        out.len = min(C, a.T - ci * C);
        return out.len > 0;
    }
    if (gc >= a.coff[a.N]) return false;
    int lo = 0, hi = a.N;  // coff[lo] <= gc < coff[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.coff[mid] <= gc) lo = mid; else hi = mid;
    }
    const int s = clampi(a.cu[lo], 0, a.T);
    const int e = clampi(a.cu[lo + 1], s, a.T);
    out.seq = lo;
    out.tok0 = s + (gc - a.coff[lo]) * C;
    out.len = min(C, e - out.tok0);
    return out.len > 0;
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-chunk work.  LDS layout (byte offsets), padded rows.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int C>
struct IntraLds {
    static constexpr int PT = 16 / sizeof(T);  // 16-byte row pad, in elements
    static constexpr int G_LD = DK + 4;        // fp32 Gam       [C][DK]
    static constexpr int K_LD = DK + PT;       // k, q           [C][DK]
    static constexpr int KT_LD = C + PT;       // transposed ops [DK|DV][C]
    static constexpr int A_LD = C + 4;         // fp32 A, L      [C][C]
    static constexpr int P_LD = C + PT;        // P              [C][C]
    static constexpr int Y_LD = 20;            // fp32 16x16 scratch
    static constexpr size_t oG = 0;
    static constexpr size_t oK = oG + size_t(C) * G_LD * 4;
    static constexpr size_t oQ = oK + size_t(C) * K_LD * sizeof(T);
    static constexpr size_t oB = oQ + size_t(C) * K_LD * sizeof(T);
    static constexpr size_t oKT = oB + size_t(C) * 4;
    static constexpr size_t oVT = oKT + size_t(DK) * KT_LD * sizeof(T);
    static constexpr size_t oA = oVT + size_t(DV) * KT_LD * sizeof(T);
    static constexpr size_t oL = oA + size_t(C) * A_LD * 4;
    static constexpr size_t oP = oL + size_t(C) * A_LD * 4;
    static constexpr size_t oY = oP + size_t(C) * P_LD * sizeof(T);
    static constexpr size_t bytes = oY + size_t(3) * 16 * Y_LD * 4;
};

template <class T, int DK, int DV, int C>
__global__ __launch_bounds__(kThreads) void kda_intra_kernel(PrefillArgs a) {
    using Ly = IntraLds<T, DK, DV, C>;
    using M = Mma<T>;
    typedef typename M::Frag Frag;
    constexpr int NT = C / kTile;
    constexpr int G_LD = Ly::G_LD, K_LD = Ly::K_LD, KT_LD = Ly::KT_LD;
    constexpr int A_LD = Ly::A_LD, P_LD = Ly::P_LD, Y_LD = Ly::Y_LD;
    constexpr int EV = 16 / sizeof(T);  // elements per 16-byte vector

    extern __shared__ __align__(16) unsigned char smem[];
    float *sG = reinterpret_cast<float *>(smem + Ly::oG);
    T *sK = reinterpret_cast<T *>(smem + Ly::oK);
    T *sQ = reinterpret_cast<T *>(smem + Ly::oQ);
    float *sB = reinterpret_cast<float *>(smem + Ly::oB);
    T *sKT = reinterpret_cast<T *>(smem + Ly::oKT);  // beta k e^Gam ^T, later W^T
    T *sVT = reinterpret_cast<T *>(smem + Ly::oVT);  // beta v ^T,       later Ut^T
    float *sA = reinterpret_cast<float *>(smem + Ly::oA);
    float *sL = reinterpret_cast<float *>(smem + Ly::oL);
    T *sP = reinterpret_cast<T *>(smem + Ly::oP);
    float *sY = reinterpret_cast<float *>(smem + Ly::oY);

    const int gc = blockIdx.x, h = blockIdx.y;
    ChunkLoc loc;
    if (!locate_chunk(a, gc, C, loc)) return;  // uniform over the workgroup
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int H = a.H;
    const T *qg = static_cast<const T *>(a.q);
    const T *kg = static_cast<const T *>(a.k);
    const T *vg = static_cast<const T *>(a.v);
    const size_t slot = size_t(gc) * H + h;

    // ---- phase 0: stage g, k, q, beta (tail rows are neutral: zeros) ----
    for (int t = tid; t < C; t += kThreads)
        sB[t] = (t < loc.len) ? a.beta[size_t(loc.tok0 + t) * H + h] : 0.f;
    constexpr int GV = DK / 4;
    for (int i = tid; i < C * GV; i += kThreads) {
        const int t = i / GV, cv = i - t * GV;
        float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
        if (t < loc.len)
            x = *reinterpret_cast<const float4 *>(a.g + (size_t(loc.tok0 + t) * H + h) * DK + cv * 4);
        *reinterpret_cast<float4 *>(sG + t * G_LD + cv * 4) = x;
    }
    constexpr int KV = DK / EV;
    for (int i = tid; i < C * KV; i += kThreads) {
        const int t = i / KV, cv = i - t * KV;
        uint4 xk = make_uint4(0, 0, 0, 0), xq = make_uint4(0, 0, 0, 0);
        if (t < loc.len) {
            const size_t off = (size_t(loc.tok0 + t) * H + h) * DK + cv * EV;
            xk = *reinterpret_cast<const uint4 *>(kg + off);
            xq = *reinterpret_cast<const uint4 *>(qg + off);
        }
        *reinterpret_cast<uint4 *>(sK + t * K_LD + cv * EV) = xk;
        *reinterpret_cast<uint4 *>(sQ + t * K_LD + cv * EV) = xq;
    }
    for (int i = tid; i < C * A_LD; i += kThreads) sL[i] = 0.f;
    __syncthreads();

    // ---- phase 1: Gam = cumulative log-decay along the chunk, per channel --
    {
        constexpr int TPC = kThreads / DK;  // threads per channel
        constexpr int SL = C / TPC;         // rows per thread
        static_assert(TPC * DK == kThreads && SL >= 1, "cumsum split");
        const int c = tid % DK, seg = tid / DK;
        float run = 0.f;
#pragma unroll
        for (int r = 0; r < SL; ++r) {
            float *p = sG + (seg * SL + r) * G_LD + c;
            run += *p;
            *p = run;
        }
        float *sTot = sA;  // scratch until phase 3
        sTot[seg * DK + c] = run;
        __syncthreads();
        float off = 0.f;
        for (int s = 0; s < seg; ++s) off += sTot[s * DK + c];
        if (seg > 0) {
#pragma unroll
            for (int r = 0; r < SL; ++r) sG[(seg * SL + r) * G_LD + c] += off;
        }
        __syncthreads();
    }

    // ---- phase 2: elementwise operands ----
    // beta_s k_s e^{Gam_s}, transposed: B operand of W = L (beta k e^Gam)
    for (int i = tid; i < C * DK; i += kThreads) {
        const int s = i % C, c = i / C;
        const float x = sB[s] * to_f32(sK[s * K_LD + c]) * exp_e(sG[s * G_LD + c]);
        sKT[c * KT_LD + s] = from_f32<T>(x);
    }
    // beta_s v_s, transposed: B operand of Ut = L (beta v)
    constexpr int VV = DV / EV;
    for (int i = tid; i < C * VV; i += kThreads) {
        const int s = i / VV, jv = i - s * VV;
        Vec16<T> x;
        x.raw = make_uint4(0, 0, 0, 0);
        if (s < loc.len)
            x.raw = *reinterpret_cast<const uint4 *>(vg + (size_t(loc.tok0 + s) * H + h) * DV + jv * EV);
        const float bs = sB[s];
#pragma unroll
        for (int e = 0; e < EV; ++e) sVT[(jv * EV + e) * KT_LD + s] = from_f32<T>(bs * x.get(e));
    }
    // (k e^{Gam_last - Gam})^T and e^{Gam_last} for the state update
    {
        T *KtT = static_cast<T *>(a.KtT) + slot * DK * C;
        constexpr int TV = C / EV;
        for (int i = tid; i < DK * TV; i += kThreads) {
            const int c = i / TV, tv = i - c * TV;
            const float glast = sG[(C - 1) * G_LD + c];
            Vec16<T> out;
            T *po = reinterpret_cast<T *>(&out.raw);
#pragma unroll
            for (int e = 0; e < EV; ++e) {
                const int t = tv * EV + e;
                po[e] = from_f32<T>(to_f32(sK[t * K_LD + c]) * exp_e(glast - sG[t * G_LD + c]));
            }
            *reinterpret_cast<uint4 *>(KtT + size_t(c) * C + tv * EV) = out.raw;
        }
        if (tid < DK) a.D[slot * DK + tid] = exp_e(sG[(C - 1) * G_LD + tid]);
    }

    // ---- phase 3: A (strictly lower, row-scaled by beta) and P (lower incl.)
    //      on MFMA, one 16x16 tile pair (I, J <= I) at a time ----
    constexpr int NPAIR = NT * (NT + 1) / 2;
    for (int item = wid; item < NPAIR; item += kWaves) {
        int I = 0, rem = item;
        while (rem > I) { rem -= I + 1; ++I; }
        const int J = rem;
        const int row = kTile * I + l16;  // token t of the A fragment
        const int col = kTile * J + l16;  // token s of the B fragment
        const float *gref = sG + (I > 0 ? kTile * I - 1 : 0) * G_LD;  // r_I: row before tile I
        floatx4 accA = zero4(), accP = zero4();
#pragma unroll
        for (int kk = 0; kk < DK / M::K; ++kk) {
            Frag fk, fq, fb;
#pragma unroll
            for (int j = 0; j < M::KPL; ++j) {
                const int c = kk * M::K + grp * M::KPL + j;
                const float r = (I > 0) ? gref[c] : 0.f;
                const float ea = exp_e(sG[row * G_LD + c] - r);  // <= 1
                const float eb = exp_e(r - sG[col * G_LD + c]);  // <= e^80
                M::set(fk, j, to_f32(sK[row * K_LD + c]) * ea);
                M::set(fq, j, to_f32(sQ[row * K_LD + c]) * ea);
                M::set(fb, j, to_f32(sK[col * K_LD + c]) * eb);
            }
            accA = M::mma(fk, fb, accA);
            accP = M::mma(fq, fb, accP);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = kTile * I + 4 * grp + r;
            sA[t * A_LD + col] = (col < t) ? sB[t] * accA[r] : 0.f;
            sP[t * P_LD + col] = from_f32<T>((col <= t) ? accP[r] : 0.f);
        }
    }
    for (int i = tid; i < C * C; i += kThreads) {  // tiles above the diagonal
        const int t = i / C, s = i - t * C;
        if ((s >> 4) > (t >> 4)) {
            sA[t * A_LD + s] = 0.f;
            sP[t * P_LD + s] = from_f32<T>(0.f);
        }
    }
    __syncthreads();

    // ---- phase 4: L = (I + A)^-1 by blocked forward substitution (fp32) ----
    // 4a: the NT diagonal 16x16 blocks, one column per lane (wave 0)
    if (wid == 0) {
        const int b = lane >> 4, colx = lane & 15;
        if (b < NT) {
            const float *Ab = sA + (kTile * b) * A_LD + kTile * b;
            float X[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = (i == colx) ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= Ab[i * A_LD + j] * X[j];
                X[i] = acc;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) sL[(kTile * b + i) * A_LD + kTile * b + colx] = X[i];
        }
    }
    __syncthreads();
    // 4b: off-diagonal blocks by distance d from the diagonal:
    //     L_IJ = -L_II * sum_{K=J}^{I-1} A_IK L_KJ
    for (int d = 1; d < NT; ++d) {
        const int nitems = NT - d;
        if (wid < nitems) {
            const int I = d + wid, J = wid;
            floatx4 acc = zero4();
            for (int K = J; K < I; ++K) {
#pragma unroll
                for (int kk = 0; kk < 4; ++kk) {
                    const float af = sA[(kTile * I + l16) * A_LD + kTile * K + 4 * kk + grp];
                    const float bf = sL[(kTile * K + 4 * kk + grp) * A_LD + kTile * J + l16];
                    acc = mma_f32(af, bf, acc);
                }
            }
            float *Y = sY + wid * 16 * Y_LD;
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[(4 * grp + r) * Y_LD + l16] = acc[r];
        }
        __syncthreads();
        if (wid < nitems) {
            const int I = d + wid, J = wid;
            const float *Y = sY + wid * 16 * Y_LD;
            floatx4 acc = zero4();
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float af = sL[(kTile * I + l16) * A_LD + kTile * I + 4 * kk + grp];
                const float bf = Y[(4 * kk + grp) * Y_LD + l16];
                acc = mma_f32(af, bf, acc);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) sL[(kTile * I + 4 * grp + r) * A_LD + kTile * J + l16] = -acc[r];
        }
        __syncthreads();
    }

    // ---- phase 5: W = L (beta k e^Gam), Ut = L (beta v) ----
    constexpr int NCK = DK / kTile, NCV = DV / kTile;
    constexpr int NITEM = NT * (NCK + NCV);
    constexpr int IPW = (NITEM + kWaves - 1) / kWaves;
    constexpr int KSTEPS = (C + M::K - 1) / M::K;
    floatx4 res[IPW];
#pragma unroll
    for (int it = 0; it < IPW; ++it) {
        const int item = wid + kWaves * it;
        res[it] = zero4();
        if (item < NITEM) {
            const int I = item % NT, n = item / NT;
            const T *Bop = (n < NCK) ? sKT + (kTile * n) * KT_LD : sVT + (kTile * (n - NCK)) * KT_LD;
            const int ks = min(KSTEPS, (kTile * (I + 1) + M::K - 1) / M::K);
            floatx4 acc = zero4();
            for (int kk = 0; kk < ks; ++kk) {
                const int kb = kk * M::K + grp * M::KPL;
                Frag af, bf;
                if (kb < C) {
                    af = M::load_f32(sL + (kTile * I + l16) * A_LD + kb);
                    bf = M::load(Bop + l16 * KT_LD + kb);
                } else {
                    af = Frag{};
                    bf = Frag{};
                }
                acc = M::mma(af, bf, acc);
            }
            res[it] = acc;
        }
    }
    __syncthreads();  // every read of the beta k e^Gam / beta v operands is done
    {
        T *Wg = static_cast<T *>(a.W) + slot * C * DK;
        T *Ug = static_cast<T *>(a.Ut) + slot * C * DV;
#pragma unroll
        for (int it = 0; it < IPW; ++it) {
            const int item = wid + kWaves * it;
            if (item < NITEM) {
                const int I = item % NT, n = item / NT;
                const bool isW = n < NCK;
                const int cc = kTile * (isW ? n : n - NCK) + l16;
                const int t0 = kTile * I + 4 * grp;
                const floatx4 acc = res[it];
                store4((isW ? sKT : sVT) + cc * KT_LD + t0, acc[0], acc[1], acc[2], acc[3]);
                T *dst = isW ? Wg : Ug;
                const int ld = isW ? DK : DV;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[size_t(t0 + r) * ld + cc] = from_f32<T>(acc[r]);
            }
        }
    }
    __syncthreads();

    // ---- phase 6: Q' = q e^Gam - P W and Oi = P Ut ----
    {
        T *Qg = static_cast<T *>(a.Qp) + slot * C * DK;
        T *Og = static_cast<T *>(a.Oi) + slot * C * DV;
#pragma unroll
        for (int it = 0; it < IPW; ++it) {
            const int item = wid + kWaves * it;
            if (item < NITEM) {
                const int I = item % NT, n = item / NT;
                const bool isW = n < NCK;
                const T *Bop = isW ? sKT + (kTile * n) * KT_LD : sVT + (kTile * (n - NCK)) * KT_LD;
                const int ks = min(KSTEPS, (kTile * (I + 1) + M::K - 1) / M::K);
                floatx4 acc = zero4();
                for (int kk = 0; kk < ks; ++kk) {
                    const int kb = kk * M::K + grp * M::KPL;
                    Frag af, bf;
                    if (kb < C) {
                        af = M::load(sP + (kTile * I + l16) * P_LD + kb);
                        bf = M::load(Bop + l16 * KT_LD + kb);
                    } else {
                        af = Frag{};
                        bf = Frag{};
                    }
                    acc = M::mma(af, bf, acc);
                }
                const int cc = kTile * (isW ? n : n - NCK) + l16;
                const int t0 = kTile * I + 4 * grp;
                if (isW) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int t = t0 + r;
                        const float qgam = to_f32(sQ[t * K_LD + cc]) * exp_e(sG[t * G_LD + cc]);
                        Qg[size_t(t) * DK + cc] = from_f32<T>(qgam - acc[r]);
                    }
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) Og[size_t(t0 + r) * DV + cc] = from_f32<T>(acc[r]);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state propagation over chunks, with the output fused in.
// One workgroup per (sequence, head, block of BV value columns).
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int C, int BV>
__global__ __launch_bounds__(kThreads) void kda_inter_kernel(PrefillArgs a) {
    using M = Mma<T>;
    typedef typename M::Frag Frag;
    constexpr int NT = C / kTile, NB = DV / BV, NCT = BV / kTile, NRT = DK / kTile;
    constexpr int PT = 16 / sizeof(T);
    constexpr int ST_LD = DK + PT;  // S^T as operand  [BV][DK]
    constexpr int UT_LD = C + PT;   // U^T as operand  [BV][C]
    constexpr int KSC = (C + M::K - 1) / M::K;
    __shared__ __align__(16) T sST[BV * ST_LD];
    __shared__ __align__(16) T sUT[BV * UT_LD];

    const int H = a.H;
    const int nchains = a.N * H;
    const int wg = blockIdx.x;
    int chain, blk;
    if ((nchains & 7) == 0) {
        // the NB blocks of one (sequence, head) share an XCD (and its L2):
        // workgroups are dealt round-robin to the 8 XCDs by linear id
        const int xcd = wg & 7, slot = wg >> 3;
        blk = slot % NB;
        chain = xcd + 8 * (slot / NB);
    } else {
        chain = wg / NB;
        blk = wg - chain * NB;
    }
    const int n = chain / H, h = chain - n * H;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int jb = blk * BV;

    int c_begin, c_end, tok_start, tok_end;
    if (!a.cu) {
        c_begin = n * a.nc_seq;
        c_end = c_begin + a.nc_seq;
        tok_start = n * a.T;
        tok_end = tok_start + a.T;
    } else {
        c_begin = min(a.coff[n], a.nc_max);
        c_end = min(max(a.coff[n + 1], c_begin), a.nc_max);
        tok_start = clampi(a.cu[n], 0, a.T);
        tok_end = clampi(a.cu[n + 1], tok_start, a.T);
    }

    // state tiles (m, nn): rows 16m.., value columns jb + 16nn..; wave-owned
    constexpr int NSI = NRT * NCT;
    constexpr int SPW = (NSI + kWaves - 1) / kWaves;
    constexpr int NXI = NT * NCT;
    constexpr int XPW = (NXI + kWaves - 1) / kWaves;
    floatx4 S[SPW];
    const size_t sbase = size_t(chain) * DK * DV;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int item = wid + kWaves * i;
        S[i] = zero4();
        if (item < NSI && a.h0) {
            const int m = item % NRT, nn = item / NRT;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                S[i][r] = a.h0[sbase + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16];
        }
    }

    T *og = static_cast<T *>(a.o);
    for (int gc = c_begin; gc < c_end; ++gc) {
        const int tok0 = tok_start + (gc - c_begin) * C;
        const int len = min(C, tok_end - tok0);
        const size_t slot = size_t(gc) * H + h;
        const T *W = static_cast<const T *>(a.W) + slot * C * DK;
        const T *Qp = static_cast<const T *>(a.Qp) + slot * C * DK;
        const T *KtT = static_cast<const T *>(a.KtT) + slot * DK * C;
        const T *Ut = static_cast<const T *>(a.Ut) + slot * C * DV;
        const T *Oi = static_cast<const T *>(a.Oi) + slot * C * DV;
        const float *D = a.D + slot * DK;

        // 1. S^T -> LDS in the operand dtype
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT, nn = item / NRT;
                store4(sST + (kTile * nn + l16) * ST_LD + kTile * m + 4 * grp, S[i][0], S[i][1], S[i][2], S[i][3]);
            }
        }
        __syncthreads();

        // 2. X = W S and O = Q' S; U = Ut - X -> LDS; o = Oi + O
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NXI) {
                const int I = item % NT, nn = item / NT;
                floatx4 ax = zero4(), ao = zero4();
#pragma unroll
                for (int kk = 0; kk < DK / M::K; ++kk) {
                    const int kb = kk * M::K + grp * M::KPL;
                    const Frag wf = M::load(W + (kTile * I + l16) * DK + kb);
                    const Frag qf = M::load(Qp + (kTile * I + l16) * DK + kb);
                    const Frag sf = M::load(sST + (kTile * nn + l16) * ST_LD + kb);
                    ax = M::mma(wf, sf, ax);
                    ao = M::mma(qf, sf, ao);
                }
                const int j = jb + kTile * nn + l16;
                const int t0 = kTile * I + 4 * grp;
                float u[4];
#pragma unroll
                for (int r = 0; r < 4; ++r) u[r] = to_f32(Ut[size_t(t0 + r) * DV + j]) - ax[r];
                store4(sUT + (kTile * nn + l16) * UT_LD + t0, u[0], u[1], u[2], u[3]);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (t0 + r < len)
                        og[(size_t(tok0 + t0 + r) * H + h) * DV + j] =
                            from_f32<T>(to_f32(Oi[size_t(t0 + r) * DV + j]) + ao[r]);
            }
        }
        __syncthreads();

        // 3. S = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT, nn = item / NRT;
                floatx4 acc = S[i];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[r] *= D[kTile * m + 4 * grp + r];
#pragma unroll
                for (int kk = 0; kk < KSC; ++kk) {
                    const int kb = kk * M::K + grp * M::KPL;
                    Frag af, bf;
                    if (kb < C) {
                        af = M::load(KtT + (kTile * m + l16) * C + kb);
                        bf = M::load(sUT + (kTile * nn + l16) * UT_LD + kb);
                    } else {
                        af = Frag{};
                        bf = Frag{};
                    }
                    acc = M::mma(af, bf, acc);
                }
                S[i] = acc;
            }
        }
    }

    if (a.ht) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT, nn = item / NRT;
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    a.ht[sbase + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16] = S[i][r];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host-side launch of one (dtype, dk, dv, chunk, bv) instance.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int C, int BV>
hipError_t launch_prefill_instance(const PrefillArgs &a, hipStream_t s) {
    using Ly = IntraLds<T, DK, DV, C>;
    static_assert(Ly::bytes <= 160 * 1024, "intra-chunk LDS exceeds 160 KiB");
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&kda_intra_kernel<T, DK, DV, C>),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, int(Ly::bytes));
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    if (a.nc_max > 0) {
        prof_begin(s);
        hipLaunchKernelGGL((kda_intra_kernel<T, DK, DV, C>), dim3(a.nc_max, a.H), dim3(kThreads),
                           Ly::bytes, s, a);
        prof_end(s, "kda_intra");
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int nwg = a.N * a.H * (DV / BV);
    if (nwg > 0) {
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, DV, C, BV>), dim3(nwg), dim3(kThreads), 0, s, a);
        prof_end(s, "kda_inter");
    }
    return hipGetLastError();
}

}  // namespace kda
