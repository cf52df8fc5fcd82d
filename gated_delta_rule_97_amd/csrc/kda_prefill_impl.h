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
// and, sequentially over chunks, with the state kept on chip in fp32:
//   U      = Ut - W S
//   o      = (q e^Gam) S + P U
//   S_next = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U
//
// Kernel 1 (kda_intra_kernel): one workgroup per (chunk, head), fully
//   parallel; everything that does not depend on the incoming state: W, Ut,
//   q e^Gam, P, K~^T = (k e^{Gam_last - Gam})^T and e^{Gam_last}.
// Kernel 2 (kda_inter_kernel and its variants): one workgroup per
//   (sequence, head, dv block), sequential over the sequence's chunks; the
//   fp32 state block lives in MFMA accumulator registers for the whole
//   sequence.
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

// A read-only int of the chunk map or cu_seqlens, through the constant
// address space: with a wave-uniform index it becomes a scalar load, which
// does not wait behind the wave's outstanding vector stores.
__device__ __forceinline__ int ld_const(const int32_t *p, int i) {
    return ((const __attribute__((address_space(4))) int32_t *)p)[i];
}

__device__ __forceinline__ bool locate_chunk(const PrefillArgs &a, int gc, int C, ChunkLoc &out) {
    if (!a.cu) {
        const int n = fdiv(gc, a.fd_nc_seq), ci = gc - n * a.nc_seq;
        if (n >= a.N) return false;
        out.seq = n;
        out.tok0 = n * a.T + ci * C;
        out.len = min(C, a.T - ci * C);
        return out.len > 0;
    }
    if (gc >= ld_const(a.coff, a.N)) return false;
    int lo = 0, hi = a.N;  // coff[lo] <= gc < coff[hi]
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (ld_const(a.coff, mid) <= gc) lo = mid; else hi = mid;
    }
    const int s = clampi(ld_const(a.cu, lo), 0, a.T);
    const int e = clampi(ld_const(a.cu, lo + 1), s, a.T);
    out.seq = lo;
    out.tok0 = s + (gc - ld_const(a.coff, lo)) * C;
    out.len = min(C, e - out.tok0);
    return out.len > 0;
}

// Chunk slot of the intra-chunk pass's wc-th (chunk, all heads) group.  The
// chunks go in descending order of their index within the sequence
// (sequences interleaved; a packed batch simply reversed), so the operands of
// every sequence's first chunks are written last: the state pass, which
// starts there, then finds them still in the last-level cache.
__device__ __forceinline__ int intra_slot(const PrefillArgs &a, int wc) {
    if (!a.cu) {  // chunks win_c0 .. win_c0 + win_nc - 1 of this launch's sequences
        const int j = fdiv(wc, a.fd_win_nn);
        return (a.win_n0 + wc - j * a.win_nn) * a.nc_seq + (a.win_c0 + a.win_nc - 1 - j);
    }
    return a.nc_max - 1 - wc;
}

// Hand-off slot (chunk index) of the same group.  The windows of a
// fixed-length batch all use the slots of the first one (slot = sequence in
// the window x win_len + chunk in the window), so that a window's hand-off
// overwrites the previous window's while the last-level cache still holds
// it (those lines are then never written back to HBM); with one window this
// is intra_slot itself.
__device__ __forceinline__ int intra_handoff(const PrefillArgs &a, int wc) {
    if (!a.cu) {
        const int j = fdiv(wc, a.fd_win_nn);
        return (wc - j * a.win_nn) * a.win_len + (a.win_nc - 1 - j);
    }
    return a.nc_max - 1 - wc;
}

// (chunk, all heads) groups the intra-chunk pass walks in one launch
__host__ __device__ __forceinline__ int intra_groups(const PrefillArgs &a) {
    return a.cu ? a.nc_max : a.win_nn * a.win_nc;
}

// ---------------------------------------------------------------------------
// Workspace layouts.  Every intermediate is stored in the exact order its
// consumer's wavefront reads it, so that one wave-wide load instruction is
// one contiguous, fully used span (1 KiB for a bf16 operand fragment).
//
// Operand order of an [R][K] matrix used as an MFMA A (or B) operand:
// blocks of 16 rows x Mma::K columns, block (rb, kb) at index rb*(Kp/K)+kb,
// inside a block lane (row % 16) + 16 * ((k % K) / KPL) holds KPL
// consecutive k.  Kp = K rounded up to Mma::K (the pad stays unread).
// Quad order of an [R][N] matrix read elementwise at MFMA output positions:
// 16x16 tiles, tile (r/16, n/16) at index (r/16)*(N/16) + n/16, inside a
// tile lane (n % 16) + 16 * ((r % 16) / 4) holds 4 consecutive rows.
// ---------------------------------------------------------------------------
template <class T> __host__ __device__ constexpr int kpad(int K) {
    return (K + Mma<T>::K - 1) / Mma<T>::K * Mma<T>::K;
}

template <class T, int K>
__device__ __forceinline__ size_t frag_off(int r, int k) {
    using M = Mma<T>;
    constexpr unsigned KP = kpad<T>(K);
    const unsigned ur = unsigned(r), uk = unsigned(k);  // non-negative: unsigned keeps / and % cheap
    const unsigned blk = (ur >> 4) * (KP / M::K) + uk / M::K;
    const unsigned ln = (ur & 15u) + 16u * ((uk % M::K) / M::KPL);
    return size_t(blk) * (16 * M::K) + ln * M::KPL + (uk % M::KPL);
}

// four consecutive k of row r (k0 % 4 == 0) into operand order
template <class T, int K>
__device__ __forceinline__ void store_frag4(T *base, int r, int k0, float a, float b, float c, float d) {
    if constexpr (Mma<T>::KPL >= 4) {
        store4(base + frag_off<T, K>(r, k0), a, b, c, d);
    } else {
        base[frag_off<T, K>(r, k0)] = from_f32<T>(a);
        base[frag_off<T, K>(r, k0 + 1)] = from_f32<T>(b);
        base[frag_off<T, K>(r, k0 + 2)] = from_f32<T>(c);
        base[frag_off<T, K>(r, k0 + 3)] = from_f32<T>(d);
    }
}

template <int N>
__device__ __forceinline__ size_t quad_off(int tile_r, int tile_n, int lane) {
    return size_t(unsigned(tile_r) * (N / 16) + unsigned(tile_n)) * 256 + unsigned(lane) * 4;
}

// Lower-block operand order of a chunk's scores P [C][C] (zero above the
// 16-token diagonal tiles): the operand order kept only for the k-blocks a
// row tile's product reads, p_nk(I) blocks for row tile I, row tiles in
// order (score_elems values in all).  Inside a kept block the values past
// the row tile's diagonal tile are stored zeros.
template <class T> __host__ __device__ constexpr int p_nk(int I) {
    return (kTile * (I + 1) + Mma<T>::K - 1) / Mma<T>::K;
}
template <class T> __host__ __device__ constexpr int p_pre(int I) {
    int n = 0;
    for (int i = 0; i < I; ++i) n += p_nk<T>(i);
    return n;
}
template <class T, int C> __host__ __device__ constexpr int p_elems() {
    static_assert(score_elems(C, Mma<T>::K) == p_pre<T>(C / kTile) * 16 * Mma<T>::K, "score layout size");
    return p_pre<T>(C / kTile) * 16 * Mma<T>::K;
}
// four consecutive k (s0 % 4 == 0) of row t into the lower-block order
template <class T>
__device__ __forceinline__ void store_p4(T *base, int t, int s0, float a, float b, float c, float d) {
    using M = Mma<T>;
    auto off = [&](int s) -> size_t {
        const unsigned blk = unsigned(p_pre<T>(t >> 4)) + unsigned(s) / M::K;
        const unsigned ln = unsigned(t & 15) + 16u * ((unsigned(s) % M::K) / M::KPL);
        return size_t(blk) * (16 * M::K) + ln * M::KPL + (unsigned(s) % M::KPL);
    };
    if constexpr (M::KPL >= 4) {
        store4(base + off(s0), a, b, c, d);
    } else {
        base[off(s0)] = from_f32<T>(a);
        base[off(s0 + 1)] = from_f32<T>(b);
        base[off(s0 + 2)] = from_f32<T>(c);
        base[off(s0 + 3)] = from_f32<T>(d);
    }
}

// ---------------------------------------------------------------------------
// Kernel 1: intra-chunk work, persistent.  Its LDS footprint allows one
// workgroup per compute unit, so the workgroup is 16 wavefronts (four per
// SIMD) to overlap the latencies of its dependent steps.  Each workgroup
// walks (chunk, head) items chunk-major, last chunks first (intra_slot); the
// raw inputs of its next item are loaded into registers while the current
// one computes, directly in the layout their first consumer wants ("owner"
// layout):
//   g, k, q: thread (channel group cg of 4, segment sg of 4 tokens)
//   v:       thread (channel group jg of 8, segment sg of 4 tokens)
// so the cumulative decay, every decay-factored operand, the transposes and
// K~^T come out of registers in one pass, and raw inputs never touch LDS.
// ---------------------------------------------------------------------------
constexpr int kIThreads = 1024;
constexpr int kIWaves = kIThreads / kWave;
constexpr int kSR = 4;  // tokens per owner segment

template <class T, int DK, int DV, int C>
struct IntraLds {
    static constexpr int PT = 16 / sizeof(T);  // 16-byte row pad, in elements
    static constexpr int NT = C / kTile, NSEG = C / kSR, NOFF = NT * (NT - 1) / 2;
    static constexpr int K_LD = DK + PT;        // K+, K-, Q+          [C][DK]
    static constexpr int KT_LD = C + PT;        // transposed operands [DK|DV][C]
    static constexpr int A_LD = C + 4;          // fp32 A, L           [C][C]
    static constexpr int Y_LD = 20;             // fp32 16x16 tile of L^T, padded rows
    static constexpr int NLT = NT * (NT - 1) / 2;  // L^T tiles (K, J), J <= K <= NT - 2
    static constexpr size_t kKK = size_t(2) * C * K_LD * sizeof(T);  // K+ and K-
    static constexpr size_t kAL = size_t(2) * C * A_LD * 4;          // A and L (reuse K+, K-)
    static constexpr size_t sQp = size_t(C) * K_LD * sizeof(T);
    static constexpr size_t sKT = size_t(DK) * KT_LD * sizeof(T);
    static constexpr size_t sVT = size_t(DV) * KT_LD * sizeof(T);
    static constexpr size_t sTail = size_t(NLT > 0 ? NLT : 1) * 16 * Y_LD * 4 + size_t(NSEG + 1) * DK * 4 +
                                    size_t(NOFF > 0 ? NOFF : 1) * DK * 4 + size_t(NT) * DK * 4 + size_t(C) * 4;
    static constexpr size_t kKA = kKK > kAL ? kKK : kAL;
    // Compact placement, for the shapes whose plain layout exceeds the 160
    // KiB of a compute unit (fp32 with a 64-token chunk and dk or dv = 128):
    // (beta v)^T is staged after the A/P products, into the dead K+/K- space
    // behind A and L.  Same products, same values.
    static constexpr bool COMPACT = kKA + sQp + sKT + sVT + sTail > size_t(160) * 1024;
    static constexpr size_t kReg = COMPACT ? (kKK > kAL + sVT ? kKK : kAL + sVT) : kKA;
    static constexpr size_t oKp = 0;
    static constexpr size_t oKm = oKp + size_t(C) * K_LD * sizeof(T);
    static constexpr size_t oA = 0;
    static constexpr size_t oL = oA + size_t(C) * A_LD * 4;
    static constexpr size_t oQp = kReg;
    static constexpr size_t oKT = oQp + sQp;
    static constexpr size_t oVT = COMPACT ? kAL : oKT + sKT;
    static constexpr size_t oY = COMPACT ? oKT + sKT : oVT + sVT;
    static constexpr size_t oTot = oY + size_t(NLT > 0 ? NLT : 1) * 16 * Y_LD * 4;
    static constexpr size_t oF = oTot + size_t(NSEG + 1) * DK * 4;
    static constexpr size_t oR = oF + size_t(NOFF > 0 ? NOFF : 1) * DK * 4;
    static constexpr size_t oB = oR + size_t(NT) * DK * 4;
    static constexpr size_t bytes = oB + size_t(C) * 4;
};

template <class T, int DK, int DV, int C>
struct IntraRoles {
    static constexpr int NSEG = C / kSR;
    static constexpr int NG = (DK / 4) * NSEG;  // g/k/q owner threads
    static constexpr int NV = (DV / 8) * NSEG;  // v owner threads
    static_assert(NG + NV + DK <= kIThreads, "owner and scan threads");
    // raw registers: g (kSR x 16 B) + k, q (kSR rows x 4 values each) for
    // role G; v (kSR rows x 8 values) for role V
    static constexpr int GQ = kSR * 4 * 2 * int(sizeof(T)) / 16;  // 16-byte registers for k and q
    static constexpr int RAW_G = kSR + GQ;
    static constexpr int RAW_V = kSR * 8 * int(sizeof(T)) / 16;
    static constexpr int RAW = RAW_G > RAW_V ? RAW_G : RAW_V;
    // whole wavefronts per role: role branches can then be uniform
    static constexpr bool ALIGNED = NG % kWave == 0 && NV % kWave == 0;
};

// The thread index used for role tests.  When every role covers whole
// wavefronts this is the wave's first lane, read into a scalar register, so
// role branches are uniform jumps instead of lane masks: the compiler then
// sees the roles as exclusive paths (otherwise it must assume a wave runs
// one role's code after the other's, and it serialises their loads).
template <class T, int DK, int DV, int C>
__device__ __forceinline__ int role_tid(int tid) {
    if constexpr (IntraRoles<T, DK, DV, C>::ALIGNED) return __builtin_amdgcn_readfirstlane(tid);
    else return tid;
}

template <class T, int DK, int DV, int C>
struct IntraIn {
    u32x4 raw[IntraRoles<T, DK, DV, C>::RAW];  // 16 bytes each, as loaded
    int len;  // valid tokens of the chunk; rows at or past it are zeroed on use
};

// Element e of an array of 16-byte registers holding values of T, by bit
// operations on its 32-bit words (e is a constant after unrolling).  Reading
// through a T pointer instead would let the compiler split the words into
// 16-bit pieces right where they are loaded.
__device__ __forceinline__ unsigned raw_word(const u32x4 &x, int i) { return x[i]; }
template <class T>
__device__ __forceinline__ float raw_get(const u32x4 *raw, int e) {
    if constexpr (sizeof(T) == 2) {
        const unsigned w = raw_word(raw[e >> 3], (e >> 1) & 3);
        return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
    } else {
        return __uint_as_float(raw_word(raw[e >> 2], e & 3));
    }
}

// Owner coordinates: role G threads own (channel group cg of 4, segment sg),
// channel groups fastest (their row stores of K+, K-, Q+ are then contiguous
// across lanes); role V threads own (channel group jg of 8, segment sg),
// segments fastest (their only stores, the columns of (beta v)^T, are then
// contiguous across lanes).
template <class T, int DK, int DV, int C>
__device__ __forceinline__ void owner_coords(int tid, bool &is_g, int &cgrp, int &sg) {
    using R = IntraRoles<T, DK, DV, C>;
    is_g = tid < R::NG;
    const int u = is_g ? tid : tid - R::NG;
    cgrp = is_g ? u % (DK / 4) : u / R::NSEG;
    sg = is_g ? u / (DK / 4) : u % R::NSEG;
}

// Value j (0..7) of token r of a role V thread.  Registers: raw[r] holds
// the first 16 bytes of its 8 values, raw[kSR + r] the next 16 (fp32 only).
template <class T, int DK, int DV, int C>
__device__ __forceinline__ float v_get(const IntraIn<T, DK, DV, C> &in, int r, int j) {
    if constexpr (sizeof(T) == 2) return raw_get<T>(in.raw + r, j);
    else return j < 4 ? raw_get<T>(in.raw + r, j) : raw_get<T>(in.raw + kSR + r, j - 4);
}

// The G and V roles issue the same load instructions with role-selected
// addresses (a V thread's unused k/q slots re-read its own v row), and the
// loads are unconditional: rows past the chunk end re-read its last row and
// are zeroed when consumed, after intra_fence.  A per-role or per-row branch
// around the loads would make the compiler merge their registers with other
// paths and wait for the data right where it is requested.
template <class T, int DK, int DV, int C>
__device__ __forceinline__ void intra_fetch(IntraIn<T, DK, DV, C> &in, const PrefillArgs &a, const ChunkLoc &loc,
                                            int h, int tid) {
    using R = IntraRoles<T, DK, DV, C>;
    const int H = a.H;
    in.len = loc.len;
    if (role_tid<T, DK, DV, C>(tid) < R::NG + R::NV) {
        bool is_g;
        int cgrp, sg;
        owner_coords<T, DK, DV, C>(tid, is_g, cgrp, sg);
#pragma unroll
        for (int r = 0; r < kSR; ++r) {
            const int t = min(kSR * sg + r, loc.len - 1);
            const size_t row = size_t(loc.tok0 + t) * H + h;
            const char *pv = reinterpret_cast<const char *>(static_cast<const T *>(a.v) + row * DV + 8 * cgrp);
            const char *p16 = is_g ? reinterpret_cast<const char *>(a.g + row * DK + 4 * cgrp) : pv;
            const char *pk = is_g ? reinterpret_cast<const char *>(static_cast<const T *>(a.k) + row * DK + 4 * cgrp)
                                  : pv + (sizeof(T) == 4 ? 16 : 0);
            const char *pq = is_g ? reinterpret_cast<const char *>(static_cast<const T *>(a.q) + row * DK + 4 * cgrp)
                                  : pv;
            in.raw[r] = *reinterpret_cast<const u32x4 *>(p16);
            if constexpr (sizeof(T) == 2) {  // k and q: 8 bytes each, packed into one register
                // the v owners hold their 8 values in raw[r] alone: when roles
                // cover whole waves their k/q slots are never read, so those
                // waves skip the two loads (a wave-uniform branch)
                if (!R::ALIGNED || role_tid<T, DK, DV, C>(tid) < R::NG) {
                    const u32x2 kk = *reinterpret_cast<const u32x2 *>(pk);
                    const u32x2 qq = *reinterpret_cast<const u32x2 *>(pq);
                    in.raw[kSR + r] = u32x4{kk[0], kk[1], qq[0], qq[1]};
                } else {
                    in.raw[kSR + r] = u32x4{0u, 0u, 0u, 0u};
                }
            } else {
                in.raw[kSR + r] = *reinterpret_cast<const u32x4 *>(pk);
                in.raw[2 * kSR + r] = *reinterpret_cast<const u32x4 *>(pq);
            }
        }
    }
}

__device__ __forceinline__ void zero_unless(u32x4 &x, bool ok) {
    const unsigned m = ok ? ~0u : 0u;
    x &= m;
}

// Marks every prefetched input register as redefined at this point, then
// zeroes the rows past the chunk end (g = 0 keeps the cumulative decay flat
// there; k = q = v = beta = 0 removes them from every product).
template <class T, int DK, int DV, int C>
__device__ __forceinline__ void intra_fence(IntraIn<T, DK, DV, C> &in, int tid) {
    using R = IntraRoles<T, DK, DV, C>;
#pragma unroll
    for (int i = 0; i < R::RAW; ++i) asm volatile("" : "+v"(in.raw[i]));
    bool is_g;
    int cgrp, sg;
    owner_coords<T, DK, DV, C>(tid, is_g, cgrp, sg);
#pragma unroll
    for (int r = 0; r < kSR; ++r) {
        const bool ok = kSR * sg + r < in.len;
        zero_unless(in.raw[r], ok);
        zero_unless(in.raw[kSR + r], ok);
        if constexpr (sizeof(T) == 4) zero_unless(in.raw[2 * kSR + r], ok);
    }
}

// A value the compiler must treat as unknown at this point.
__device__ __forceinline__ int opaque(int x) {
    asm volatile("" : "+v"(x));
    return x;
}

// 8 consecutive fp32 values from LDS
__device__ __forceinline__ void lds_read8(const float *p, float (&x)[8]) {
    const float4 a = *reinterpret_cast<const float4 *>(p);
    const float4 b = *reinterpret_cast<const float4 *>(p + 4);
    x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
    x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// 8 consecutive values of T to LDS or global memory (16 bytes for bf16)
__device__ __forceinline__ void store8(bf16 *p, const float (&x)[8]) {
    bf16x8 v;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = static_cast<bf16>(x[i]);
    *reinterpret_cast<bf16x8 *>(p) = v;
}
__device__ __forceinline__ void store8(float *p, const float (&x)[8]) {
    store4(p, x[0], x[1], x[2], x[3]);
    store4(p + 4, x[4], x[5], x[6], x[7]);
}

// Off-diagonal blocks of block column J of L = (I + A)^-1 (fp32, one wave),
// top to bottom: L_IJ = -L_II * sum_{K=J}^{I-1} A_IK L_KJ.  The fp32 16x16x4
// products take their k in the order 4 * grp + kk, so a lane's four A values
// are one 16-byte row read and its four B values are rows 4 grp .. 4 grp + 3
// of L_KJ's column l16: for K = J one 16-byte read of the transposed
// diagonal tile in sY, for K > J exactly what the lane holds of -L_KJ from
// the product that made it (the accumulator layout), so the column's blocks
// stay in registers.  The sum Y, as the accumulator leaves it, is likewise
// the B operand of the product with L_II.
template <int J, int NT, int A_LD, int Y_LD>
__device__ __forceinline__ void inverse_column(const float *sA, float *sL, const float *sY, int grp, int l16) {
    floatx4 Lc[NT];  // rows 4 grp + r of column l16 of L_KJ, K > J
#pragma unroll
    for (int I = J + 1; I < NT; ++I) {
        floatx4 acc = zero4();
#pragma unroll
        for (int K = J; K < I; ++K) {
            const floatx4 af = *reinterpret_cast<const floatx4 *>(sA + (kTile * I + l16) * A_LD + kTile * K + 4 * grp);
            const floatx4 bf = (K == J) ? *reinterpret_cast<const floatx4 *>(sY + ((J * (J + 1)) / 2 + J) * 16 * Y_LD +
                                                                              l16 * Y_LD + 4 * grp)
                                        : Lc[K];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) acc = mma_f32(af[kk], bf[kk], acc);
        }
        const floatx4 lf = *reinterpret_cast<const floatx4 *>(sL + (kTile * I + l16) * A_LD + kTile * I + 4 * grp);
        floatx4 out = zero4();
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) out = mma_f32(lf[kk], acc[kk], out);
        Lc[I] = floatx4{-out[0], -out[1], -out[2], -out[3]};
#pragma unroll
        for (int r = 0; r < 4; ++r) sL[(kTile * I + 4 * grp + r) * A_LD + kTile * J + l16] = -out[r];
    }
}

// (beta v)^T of the chunk from a role V thread's registers: its 8 value
// columns, 4 tokens each.
template <class T, int DK, int DV, int C>
__device__ __forceinline__ void stage_bv(T *sVT, const float *sB, const IntraIn<T, DK, DV, C> &in, int tid) {
    constexpr int KT_LD = IntraLds<T, DK, DV, C>::KT_LD;
    bool is_g;
    int jg, sg;
    owner_coords<T, DK, DV, C>(tid, is_g, jg, sg);
    static_assert(kSR == 4, "four tokens' beta per owner");
    const float4 b4 = *reinterpret_cast<const float4 *>(sB + kSR * sg);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        store4(sVT + (8 * jg + j) * KT_LD + kSR * sg, b4.x * v_get(in, 0, j), b4.y * v_get(in, 1, j),
               b4.z * v_get(in, 2, j), b4.w * v_get(in, 3, j));
}

template <class T, int DK, int DV, int C>
__global__ __launch_bounds__(kIThreads) void kda_intra_kernel(PrefillArgs a) {
    using Ly = IntraLds<T, DK, DV, C>;
    using R = IntraRoles<T, DK, DV, C>;
    using In = IntraIn<T, DK, DV, C>;
    using M = Mma<T>;
    typedef typename M::Frag Frag;
    constexpr int NT = C / kTile, NSEG = Ly::NSEG;
    constexpr int K_LD = Ly::K_LD, KT_LD = Ly::KT_LD;
    constexpr int A_LD = Ly::A_LD, Y_LD = Ly::Y_LD;

    extern __shared__ __align__(16) unsigned char smem[];
    T *sKp = reinterpret_cast<T *>(smem + Ly::oKp);    // k e^{Gam - r_I}   (<= 1)
    T *sKm = reinterpret_cast<T *>(smem + Ly::oKm);    // k e^{r_I - Gam}   (<= e^80)
    T *sQp = reinterpret_cast<T *>(smem + Ly::oQp);    // q e^{Gam - r_I}   (<= 1)
    T *sKT = reinterpret_cast<T *>(smem + Ly::oKT);    // (beta k e^Gam)^T
    T *sVT = reinterpret_cast<T *>(smem + Ly::oVT);    // (beta v)^T
    float *sA = reinterpret_cast<float *>(smem + Ly::oA);
    float *sL = reinterpret_cast<float *>(smem + Ly::oL);
    float *sY = reinterpret_cast<float *>(smem + Ly::oY);
    float *sTot = reinterpret_cast<float *>(smem + Ly::oTot);  // segment decay totals (base 2), then their
                                                               // exclusive prefix     [NSEG + 1][DK]
    float *sF = reinterpret_cast<float *>(smem + Ly::oF);      // e^{r_I - r_J}, J < I    [NOFF][DK]
    float *sR = reinterpret_cast<float *>(smem + Ly::oR);      // e^{r_I}                 [NT][DK]
    float *sB = reinterpret_cast<float *>(smem + Ly::oB);

    const int H = a.H;
    const int nitems = intra_groups(a) * H;

    // first item of this workgroup with a valid chunk
    int item = blockIdx.x;
    ChunkLoc loc;
    while (item < nitems && !locate_chunk(a, intra_slot(a, fdiv(item, a.fd_H)), C, loc)) item += gridDim.x;
    if (item >= nitems) return;
    In in;
    intra_fetch(in, a, loc, item - H * fdiv(item, a.fd_H), int(threadIdx.x));
    // beta of the chunk: one value per lane of the last wave (which loads no
    // other input), staged in LDS at the top of each item
    constexpr int kBetaWave = kIWaves - 1;
    static_assert(kBetaWave * kWave >= R::NG + R::NV + DK, "the beta wave has no other input or scan role");
    static_assert(C <= kWave, "one beta value per lane");
    const bool beta_wave = __builtin_amdgcn_readfirstlane(int(threadIdx.x) >> 6) == kBetaWave;
    float bnx = 0.f;
    int blen = 0;
    if (beta_wave) {
        const int t = min(int(threadIdx.x & 63), loc.len - 1);
        bnx = a.beta[size_t(loc.tok0 + t) * H + (item - H * fdiv(item, a.fd_H))];
        blen = loc.len;
    }

    while (item < nitems) {
        // thread coordinates pass through an opaque copy each iteration, so
        // that the many per-stage LDS addresses are recomputed here instead
        // of being hoisted out of the loop and held in registers throughout
        const int tid = opaque(int(threadIdx.x)), lane = tid & 63;
        const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: tile math stays scalar
        const int grp = lane >> 4, l16 = lane & 15;
        const int wc = fdiv(item, a.fd_H), h = item - H * wc;
        const size_t slot = size_t(intra_handoff(a, wc)) * H + h;
        // The prefetched registers are consumed from here on, and only from
        // here: without this fence the compiler moves unpacking work up to
        // the loads at the end of the previous item, which then must wait
        // for them there and the prefetch hides no latency.
        intra_fence(in, tid);
        if (beta_wave) {
            asm volatile("" : "+v"(bnx));
            if (lane < C) sB[lane] = lane < blen ? bnx : 0.f;
        }

        // ---- cumulative log-decay: per-thread partial sums over kSR tokens.
        //      The decays are taken to base 2 once, in place (g log2(e)), so
        //      every factor below is one hardware exp2 of a difference ----
        const int rt = role_tid<T, DK, DV, C>(tid);
        if (rt < R::NG) {
            const int cg = tid % (DK / 4), sg = tid / (DK / 4);
            float run[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int r = 0; r < kSR; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    const float g2 = __uint_as_float(in.raw[r][c]) * kLog2e;
                    in.raw[r][c] = __float_as_uint(g2);
                    run[c] += g2;
                }
            *reinterpret_cast<float4 *>(sTot + sg * DK + 4 * cg) = make_float4(run[0], run[1], run[2], run[3]);
        }
        __syncthreads();

        // ---- exclusive prefix of the segment totals (one thread per
        //      channel), and the per-channel decay factors derived from it;
        //      meanwhile role V stages (beta v)^T ----
        if (rt >= R::NG + R::NV) {
            const int c = tid - R::NG - R::NV;
            if (c < DK) {
                float x[NSEG];
#pragma unroll
                for (int s2 = 0; s2 < NSEG; ++s2) x[s2] = sTot[s2 * DK + c];
                float run = 0.f, rr[NT];
#pragma unroll
                for (int s2 = 0; s2 < NSEG; ++s2) {
                    if (s2 % (kTile / kSR) == 0) rr[s2 / (kTile / kSR)] = run;
                    sTot[s2 * DK + c] = run;
                    run += x[s2];
                }
                sTot[NSEG * DK + c] = run;
                a.D[slot * DK + c] = exp2_hw(run);
#pragma unroll
                for (int I2 = 0; I2 < NT; ++I2) {
                    sR[I2 * DK + c] = exp2_hw(rr[I2]);
#pragma unroll
                    for (int J2 = 0; J2 < I2; ++J2) sF[(I2 * (I2 - 1) / 2 + J2) * DK + c] = exp2_hw(rr[I2] - rr[J2]);
                }
            }
        } else if (!Ly::COMPACT && rt >= R::NG) {
            stage_bv(sVT, sB, in, tid);
        }
        __syncthreads();

        // ---- decay-factored operands, transposes and K~^T, from registers:
        //      with x = Gam - r_I (<= 0 within tile I),
        //        K+ = k e^x, Q+ = q e^x, K- = k e^-x (<= e^80, the decay bound),
        //        beta k e^Gam = beta K+ e^{r_I}   (when e^{r_I} underflows, so does e^Gam),
        //        K~ = k e^{Gam_last - Gam}, its own exponential: e^-x e^{Gam_last - r_I}
        //        would lose it when the second factor underflows and the first is large ----
        if (rt < R::NG) {
            const int cg = tid % (DK / 4), sg = tid / (DK / 4), c0 = 4 * cg;
            const int I = sg / (kTile / kSR);  // 16-token tile of this segment
            const float4 off4 = *reinterpret_cast<const float4 *>(sTot + sg * DK + c0);
            const float4 rI4 = *reinterpret_cast<const float4 *>(sTot + (kTile / kSR) * I * DK + c0);
            const float4 er4 = *reinterpret_cast<const float4 *>(sR + I * DK + c0);
            const float4 gl4 = *reinterpret_cast<const float4 *>(sTot + NSEG * DK + c0);
            const float base[4] = {off4.x - rI4.x, off4.y - rI4.y, off4.z - rI4.z, off4.w - rI4.w};
            const float glr[4] = {gl4.x - rI4.x, gl4.y - rI4.y, gl4.z - rI4.z, gl4.w - rI4.w};
            const float er[4] = {er4.x, er4.y, er4.z, er4.w};
            const float4 b4 = *reinterpret_cast<const float4 *>(sB + kSR * sg);
            const float bt[4] = {b4.x, b4.y, b4.z, b4.w};
            // per channel: four tokens' beta k e^Gam and K~, for the column stores
            Col4<T> bke[4], ktv[4];
            T *Qg = static_cast<T *>(a.Qg) + slot * C * DK;
            float run[4] = {base[0], base[1], base[2], base[3]};  // Gam - r_I, token by token
#pragma unroll
            for (int r = 0; r < kSR; ++r) {
                const int t = kSR * sg + r;
                float kp[4], km[4], qp[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    run[c] += __uint_as_float(in.raw[r][c]);
                    const float x = run[c];
                    const float kv = raw_get<T>(in.raw + kSR, (sizeof(T) == 2 ? 8 * r : 4 * r) + c);
                    const float qv = sizeof(T) == 2 ? raw_get<T>(in.raw + kSR, 8 * r + 4 + c)
                                                    : raw_get<T>(in.raw + 2 * kSR, 4 * r + c);
                    const float e = exp2_hw(x);    // <= 1
                    const float ei = exp2_hw(-x);  // <= e^80
                    kp[c] = kv * e;
                    qp[c] = qv * e;
                    km[c] = kv * ei;
                    bke[c].set(r, bt[r] * er[c] * kp[c]);
                    ktv[c].set(r, kv * exp2_hw(glr[c] - x));  // <= 1
                }
                store4(sKp + t * K_LD + c0, kp[0], kp[1], kp[2], kp[3]);
                store4(sKm + t * K_LD + c0, km[0], km[1], km[2], km[3]);
                store4(sQp + t * K_LD + c0, qp[0], qp[1], qp[2], qp[3]);
                // q e^Gam = Q+ e^{r_I}, for the state pass's Q S
                store_frag4<T, DK>(Qg, t, c0, qp[0] * er[0], qp[1] * er[1], qp[2] * er[2], qp[3] * er[3]);
            }
            // channels: (beta k e^Gam)^T to LDS and K~^T to HBM, 4 tokens per store
            T *KtT = static_cast<T *>(a.KtT) + slot * DK * kpad<T>(C);
            static_assert(kSR == 4, "column stores are four tokens wide");
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                bke[c].store(sKT + (c0 + c) * KT_LD + kSR * sg);
                if constexpr (Mma<T>::KPL >= 4) {
                    ktv[c].store(KtT + frag_off<T, C>(c0 + c, kSR * sg));
                } else {
                    store_frag4<T, C>(KtT, c0 + c, kSR * sg, ktv[c].v[0], ktv[c].v[1], ktv[c].v[2], ktv[c].v[3]);
                }
            }
        }
        // the next item (its inputs are requested during the inversion below)
        const ChunkLoc cur = loc;
        int nxt = item + gridDim.x;
        while (nxt < nitems && !locate_chunk(a, intra_slot(a, fdiv(nxt, a.fd_H)), C, loc)) nxt += gridDim.x;
        if (nxt >= nitems) {  // no next item: the prefetch below (never used) reads one row
            loc = cur;
            loc.len = 1;
        }
        const int nxt_i = nxt < nitems ? nxt : item, nxt_h = nxt_i - H * fdiv(nxt_i, a.fd_H);
        __syncthreads();

        // ---- A (strictly lower, row-scaled by beta) and P (lower incl.) on
        //      MFMA, one 16x16 tile pair (I, J <= I) per wave.  Operands are
        //      K+ and Q+ of tile I and K- of tile J, times e^{r_I - r_J} when
        //      J < I; on the diagonal the column operand is <= e^80.  P is
        //      formed transposed (K- Q+^T), which leaves each lane four
        //      consecutive k of one row: the operand fragment of the state
        //      pass's P U, stored straight to HBM. ----
        constexpr int NPAIR = NT * (NT + 1) / 2;
        static_assert(NPAIR <= kIWaves, "A/P tile pairs");
        floatx4 accA = zero4(), accP = zero4();
        if (wid < NPAIR) {
            int I = 0, rem = wid;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            const int row = kTile * I + l16, col = kTile * J + l16;
            const float *fIJ = sF + (I * (I - 1) / 2 + J) * DK;
#pragma unroll 2
            for (int kk = 0; kk < DK / M::K; ++kk) {
                const int cb = kk * M::K + grp * M::KPL;
                const Frag fk = M::load(sKp + row * K_LD + cb);
                const Frag fq = M::load(sQp + row * K_LD + cb);
                Frag fb = M::load(sKm + col * K_LD + cb);
                if (J < I) {
                    if constexpr (M::KPL == 8) {
                        float f8[8];
                        lds_read8(fIJ + cb, f8);
#pragma unroll
                        for (int j = 0; j < 8; ++j) M::set(fb, j, to_f32(fb[j]) * f8[j]);
                    } else {
                        M::set(fb, 0, fb * fIJ[cb]);
                    }
                }
                accA = M::mma(fk, fb, accA);
                accP = M::mma(fb, fq, accP);
            }
            // lane: P[16 I + l16][16 J + 4 grp + r], causal on the diagonal tile
            float pv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv[r] = (J < I || 4 * grp + r <= l16) ? accP[r] : 0.f;
            store_p4<T>(static_cast<T *>(a.Ps) + slot * p_elems<T, C>(), kTile * I + l16, kTile * J + 4 * grp, pv[0],
                        pv[1], pv[2], pv[3]);
        }
        __syncthreads();  // K+ and K- are dead: their LDS becomes A and L
        static_assert(NT * NT <= kIWaves, "one tile of A/P or of the zero upper part per wave");
        if (wid >= NPAIR && wid < NT * NT) {
            // tile (row J, column I), J < I, is zero in L and P; P's zeros are
            // stored where the tile shares a kept k-block with row tile J
            int I = 1, rem = wid - NPAIR;
            while (rem >= I) { rem -= I; ++I; }
            const int J = rem, col = kTile * I + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) sL[(kTile * J + 4 * grp + r) * A_LD + col] = 0.f;
            if ((kTile * I) / M::K < p_nk<T>(J))
                store_p4<T>(static_cast<T *>(a.Ps) + slot * p_elems<T, C>(), kTile * J + l16, kTile * I + 4 * grp, 0.f,
                            0.f, 0.f, 0.f);
        }
        if (wid < NPAIR) {
            int I = 0, rem = wid;
            while (rem > I) { rem -= I + 1; ++I; }
            const int J = rem;
            const int col = kTile * J + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = kTile * I + 4 * grp + r;
                sA[t * A_LD + col] = (col < t) ? sB[t] * accA[r] : 0.f;
            }
        }
        if constexpr (Ly::COMPACT)
            if (rt >= R::NG && rt < R::NG + R::NV) stage_bv(sVT, sB, in, tid);  // into the K+/K- space
        __syncthreads();

        // ---- L = (I + A)^-1 by blocked forward substitution (fp32) on the
        //      waves that load no inputs, while the owner waves issue the next
        //      item's loads.  Wave kSolveWave + J owns block column J: it
        //      computes all diagonal blocks (the same values on every such
        //      wave), then L_IJ for I > J from its own column.  Each wave reads
        //      back only what it wrote itself (its LDS accesses complete in
        //      order), so the inverse needs no barrier of its own, and the
        //      longest chain is column 0 instead of the whole triangle ----
        constexpr int kSolveWave = (IntraRoles<T, DK, DV, C>::NG + IntraRoles<T, DK, DV, C>::NV + kWave - 1) / kWave;
        constexpr int kSolveWaves = NT > 1 ? NT - 1 : 1;
        static_assert(kSolveWave + kSolveWaves <= kIWaves, "waves with no input role");
        if (wid >= kSolveWave && wid < kSolveWave + kSolveWaves) {
            const int Jw = wid - kSolveWave;  // this wave's block column
            // the NT diagonal 16x16 blocks, one column per lane
            const int b = lane >> 4, colx = lane & 15;
            if (b < NT) {
                const float *Ab = sA + (kTile * b) * A_LD + kTile * b;
                // right-looking: once X[j] is final it is taken out of every
                // later row, so each row's sum runs over j in the same order as
                // X[i] = e_i - sum_{j<i} A_ij X[j] (the same rounding), but the
                // A values are two-column row pieces read ahead of their use
                // and the serial dependency is one FMA per row
                float X[16];
#pragma unroll
                for (int i = 0; i < 16; ++i) X[i] = (i == colx) ? 1.f : 0.f;
#pragma unroll
                for (int jb = 0; jb < 16; jb += 2) {
                    float2 ar[16];
#pragma unroll
                    for (int i = jb + 1; i < 16; ++i) ar[i] = *reinterpret_cast<const float2 *>(Ab + i * A_LD + jb);
#pragma unroll
                    for (int i = jb + 1; i < 16; ++i) X[i] -= ar[i].x * X[jb];
#pragma unroll
                    for (int i = jb + 2; i < 16; ++i) X[i] -= ar[i].y * X[jb + 1];
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) sL[(kTile * b + i) * A_LD + kTile * b + colx] = X[i];
                if (b <= NT - 2) {  // its transpose, for the off-diagonal products
                    float *t = sY + ((b * (b + 1)) / 2 + b) * 16 * Y_LD + colx * Y_LD;
#pragma unroll
                    for (int i = 0; i < 16; i += 4)
                        *reinterpret_cast<floatx4 *>(t + i) = floatx4{X[i], X[i + 1], X[i + 2], X[i + 3]};
                }
            }
            // off-diagonal blocks of column Jw, top to bottom (they read the
            // diagonal blocks other lanes of this wave wrote)
            if constexpr (NT > 1) {
                wave_lds_sync();
                if (Jw == 0) inverse_column<0, NT, A_LD, Y_LD>(sA, sL, sY, grp, l16);
                if constexpr (NT > 2) if (Jw == 1) inverse_column<1, NT, A_LD, Y_LD>(sA, sL, sY, grp, l16);
                if constexpr (NT > 3) if (Jw == 2) inverse_column<2, NT, A_LD, Y_LD>(sA, sL, sY, grp, l16);
                static_assert(NT <= 4, "three block columns at most");
            }
        }
        // ---- the next item's inputs go in flight now, beside the inverse.
        //      After the last item the loads repeat this item's (and go
        //      unused): an unconditional load keeps the registers free of
        //      merges that would wait here ----
        intra_fetch(in, a, loc, nxt_h, tid);
        if (beta_wave) {
            const int t = min(lane, loc.len - 1);
            bnx = a.beta[size_t(loc.tok0 + t) * H + nxt_h];
            blen = loc.len;
        }
        __syncthreads();

        // ---- W = L (beta k e^Gam) as W^T = (beta k e^Gam)^T L^T, so that a
        //      lane's output is four consecutive channels of one token;
        //      Ut = L (beta v).  Items: W tiles (channel tile m, token tile n),
        //      then Ut tiles (token tile I, value tile n); item wi of wave w
        //      is w + kIWaves * it, so every item of a wave has the same token
        //      tile and the L fragments are read once.  Wave-uniform branches
        //      pick the W or Ut form. ----
        constexpr int NCK = DK / kTile, NCV = DV / kTile;
        constexpr int NIW = NT * NCK, NITEM = NT * (NCK + NCV);
        constexpr int IPW = (NITEM + kIWaves - 1) / kIWaves;
        constexpr int KSTEPS = (C + M::K - 1) / M::K;
        static_assert(kIWaves % NT == 0, "a wave keeps one token tile");
        const int tt = wid % NT;
        // the k-steps past the diagonal tile multiply the zero upper tiles of
        // L: doing them keeps every operand read unconditional, so a wave
        // issues all its LDS reads before its first product
        // k-fragment kk of a row starting at p; zero past the chunk (when C < K)
        auto frag_at = [&](const T *p, int kk) -> Frag {
            const int kb = kk * M::K + grp * M::KPL;
            return (C % M::K == 0 || kb < C) ? M::load(p + kb) : Frag{};
        };
        floatx4 res[IPW];
        {
            Frag lf[KSTEPS];
#pragma unroll
            for (int kk = 0; kk < KSTEPS; ++kk) {
                const int kb = kk * M::K + grp * M::KPL;
                lf[kk] = (C % M::K == 0 || kb < C) ? M::load_f32(sL + (kTile * tt + l16) * A_LD + kb) : Frag{};
            }
#pragma unroll
            for (int it = 0; it < IPW; ++it) {
                const int wi = wid + kIWaves * it;
                floatx4 acc = zero4();
                if (wi < NIW) {
                    const T *ob = sKT + (kTile * (wi / NT) + l16) * KT_LD;
#pragma unroll
                    for (int kk = 0; kk < KSTEPS; ++kk)
                        acc = M::mma(frag_at(ob, kk), lf[kk], acc);
                } else if (wi < NITEM) {
                    const T *ob = sVT + (kTile * ((wi - NIW) / NT) + l16) * KT_LD;
#pragma unroll
                    for (int kk = 0; kk < KSTEPS; ++kk)
                        acc = M::mma(lf[kk], frag_at(ob, kk), acc);
                }
                res[it] = acc;
            }
        }
        // W and Ut to HBM, in their consumers' orders.  No LDS is written
        // after the products: the next item's first writes (segment totals,
        // beta) touch nothing they read, and its first barrier orders the rest.
        {
            T *Wg = static_cast<T *>(a.W) + slot * C * DK;
            T *Ug = static_cast<T *>(a.Ut) + slot * C * DV;
#pragma unroll
            for (int it = 0; it < IPW; ++it) {
                const int wi = wid + kIWaves * it;
                const floatx4 acc = res[it];
                if (wi < NIW) {
                    // lane holds W[t][c0..c0+3]: t = 16 tt + l16, c0 = 16 m + 4 grp
                    const int t = kTile * tt + l16, c0 = kTile * (wi / NT) + 4 * grp;
                    store_frag4<T, DK>(Wg, t, c0, acc[0], acc[1], acc[2], acc[3]);
                } else if (wi < NITEM) {
                    // lane holds Ut[t0..t0+3][j]: t0 = 16 tt + 4 grp, j = 16 n + l16
                    store4(Ug + quad_off<DV>(tt, (wi - NIW) / NT, lane), acc[0], acc[1], acc[2], acc[3]);
                }
            }
        }
        item = nxt;
    }
}

// ---------------------------------------------------------------------------
// Kernel 2: state propagation over chunks, with the output fused in.
// One workgroup per (sequence, head, block of BV value columns).  The chain
// over chunks is serial, so every operand of chunk c + NS - 1 is requested
// while chunk c computes (a ring of NS register stages): the per-chunk cost
// is then the MFMA work and two LDS round trips, not the HBM latency.
// ---------------------------------------------------------------------------
template <class T> struct Quad;  // four consecutive values of T, as floats
template <> struct Quad<bf16> {
    bf16x4 v;
    __device__ __forceinline__ void load(const bf16 *p) { v = *reinterpret_cast<const bf16x4 *>(p); }
    __device__ __forceinline__ float operator[](int i) const { return static_cast<float>(v[i]); }
};
template <> struct Quad<float> {
    floatx4 v;
    __device__ __forceinline__ void load(const float *p) { v = *reinterpret_cast<const floatx4 *>(p); }
    __device__ __forceinline__ float operator[](int i) const { return v[i]; }
};

// What one state-chain launch computes.  FULL: outputs o and the state
// (ht or a checkpoint).  SUM_B: a segment's end state from a zero start, no
// outputs.  SUM_M: a segment's transition, the chain applied to an identity
// block with no value input (U = -W S), no outputs; instanced with DV = DK.
// kSumBM (accumulator-resident chain only, dk == dv): both segment summaries
// in one pass, the first half of the waves carrying B and the second half M,
// all of them on the same staged chunk operands.
enum InterMode { kFull = 0, kSumB = 1, kSumM = 2, kSumBM = 3 };

template <class T, int DK, int DV, int C, int BV>
struct InterCfg {
    typedef typename Mma<T>::Frag Frag;
    static constexpr int NT = C / kTile, NB = DV / BV, NCT = BV / kTile, NRT = DK / kTile;
    static constexpr int KSD = DK / Mma<T>::K;                  // k-steps over dk
    static constexpr int KSC = (C + Mma<T>::K - 1) / Mma<T>::K;  // k-steps over the chunk
    static constexpr int NSI = NRT * NCT;                        // state tiles
    static constexpr int SPW = (NSI + kWaves - 1) / kWaves;
    static constexpr int NXI = NT * NCT;                         // output tiles
    static constexpr int XPW = (NXI + kWaves - 1) / kWaves;
    static constexpr int NS = BV >= 32 ? 2 : 3;                  // register stages
};

// Operands of one chunk, as held by one lane.
template <class T, int DK, int DV, int C, int BV>
struct InterStage {
    using Cfg = InterCfg<T, DK, DV, C, BV>;
    typename Cfg::Frag w[Cfg::KSD], q[Cfg::KSD];   // rows of W and q e^Gam of this wave's row tile
    typename Cfg::Frag kt[Cfg::SPW][Cfg::KSC];     // rows of (k e^{Gam_last-Gam})^T per state tile
    typename Cfg::Frag pf[Cfg::KSC];               // rows of P of this wave's row tile (zero past its blocks)
    floatx4 d[Cfg::SPW];                           // e^{Gam_last} per state-tile row
    Quad<T> ut[Cfg::XPW];                          // Ut at this lane's output positions
};

template <class T, int DK, int DV, int C, int BV, int MODE>
__device__ __forceinline__ void inter_load(InterStage<T, DK, DV, C, BV> &st, const PrefillArgs &a, int gc,
                                           int h, int wid, int grp, int l16, int jb) {
    using Cfg = InterCfg<T, DK, DV, C, BV>;
    using M = Mma<T>;
    const size_t slot = size_t(gc) * a.H + h;
    const T *W = static_cast<const T *>(a.W) + slot * C * DK;
    const T *Qg = static_cast<const T *>(a.Qg) + slot * C * DK;
    const T *KtT = static_cast<const T *>(a.KtT) + slot * DK * kpad<T>(C);
    const T *UtT = static_cast<const T *>(a.Ut) + slot * C * DV;  // quad order
    const T *Ps = static_cast<const T *>(a.Ps) + slot * p_elems<T, C>();
    const float *D = a.D + slot * DK;
    const int I = wid % Cfg::NT;  // this wave's output row tile
    const int lane = l16 + 16 * grp;
#pragma unroll
    for (int kk = 0; kk < Cfg::KSD; ++kk) {
        const size_t off = size_t(I * Cfg::KSD + kk) * (16 * M::K) + lane * M::KPL;
        st.w[kk] = M::load(W + off);
        if (MODE == kFull) st.q[kk] = M::load(Qg + off);
    }
    if (MODE == kFull) {
#pragma unroll
        for (int kk = 0; kk < Cfg::KSC; ++kk) {
            const int kb = kk * M::K + grp * M::KPL;
            st.pf[kk] = (kk < p_nk<T>(I) && kb < C)
                            ? M::load(Ps + size_t(p_pre<T>(I) + kk) * (16 * M::K) + lane * M::KPL)
                            : typename Cfg::Frag{};
        }
    }
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
        const int item = wid + kWaves * i;
        if (item < Cfg::NSI) {
            const int m = item % Cfg::NRT;
#pragma unroll
            for (int kk = 0; kk < Cfg::KSC; ++kk) {
                const int kb = kk * M::K + grp * M::KPL;
                st.kt[i][kk] = (kb < C) ? M::load(KtT + size_t(m * Cfg::KSC + kk) * (16 * M::K) + lane * M::KPL)
                                        : typename Cfg::Frag{};
            }
            st.d[i] = *reinterpret_cast<const floatx4 *>(D + kTile * m + 4 * grp);
        }
    }
#pragma unroll
    for (int i = 0; i < Cfg::XPW; ++i) {
        const int item = wid + kWaves * i;
        if (item < Cfg::NXI) {
            const int nn = item / Cfg::NT;
            if (MODE != kSumM) st.ut[i].load(UtT + quad_off<DV>(I, jb / kTile + nn, lane));
        }
    }
}

// One chunk of the chain for one workgroup: S (fp32, in registers) -> o rows
// of this chunk and the next state.  ``len`` < C only on a sequence's last
// chunk; rows past it are written to a dummy area instead of o (a select,
// not a branch, so that no prefetched operand gets sunk into a branch).
template <class T, int DK, int DV, int C, int BV, int MODE>
__device__ __forceinline__ void inter_chunk(const InterStage<T, DK, DV, C, BV> &cur, floatx4 (&S)[InterCfg<T, DK, DV, C, BV>::SPW],
                                            T *sST, T *sUT, T *og, T *dummy, int tok0, int len, int H, int h,
                                            int wid, int grp, int l16, int jb) {
    using M = Mma<T>;
    using Cfg = InterCfg<T, DK, DV, C, BV>;
    typedef typename M::Frag Frag;
    constexpr int NT = Cfg::NT, NRT = Cfg::NRT, NSI = Cfg::NSI, SPW = Cfg::SPW, NXI = Cfg::NXI, XPW = Cfg::XPW;
    constexpr int PT = 16 / sizeof(T);
    constexpr int ST_LD = DK + PT, UT_LD = C + PT;
    const int I = wid % NT;

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

    // 2. X = W S and O = (q e^Gam) S; U = Ut - X -> LDS
    floatx4 oacc[XPW];
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
        const int item = wid + kWaves * i;
        oacc[i] = zero4();
        if (item < NXI) {
            const int nn = item / NT;
            floatx4 ax = zero4(), ao = zero4();
#pragma unroll
            for (int kk = 0; kk < Cfg::KSD; ++kk) {
                const int kb = kk * M::K + grp * M::KPL;
                const Frag sf = M::load(sST + (kTile * nn + l16) * ST_LD + kb);
                ax = M::mma(cur.w[kk], sf, ax);
                if (MODE == kFull) ao = M::mma(cur.q[kk], sf, ao);
            }
            const int t0 = kTile * I + 4 * grp;
            if (MODE == kSumM) {
                store4(sUT + (kTile * nn + l16) * UT_LD + t0, -ax[0], -ax[1], -ax[2], -ax[3]);
            } else {
                store4(sUT + (kTile * nn + l16) * UT_LD + t0, cur.ut[i][0] - ax[0], cur.ut[i][1] - ax[1],
                       cur.ut[i][2] - ax[2], cur.ut[i][3] - ax[3]);
            }
            oacc[i] = ao;
        }
    }
    __syncthreads();

    // o = (q e^Gam) S + P U, P's k-blocks up to this row tile's diagonal
    if (MODE == kFull) {
#pragma unroll
        for (int i = 0; i < XPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NXI) {
                const int nn = item / NT;
                floatx4 acc = oacc[i];
#pragma unroll
                for (int kk = 0; kk < Cfg::KSC; ++kk) {
                    if (kk < p_nk<T>(I)) {
                        const int kb = kk * M::K + grp * M::KPL;
                        const Frag bf = (kb < C) ? M::load(sUT + (kTile * nn + l16) * UT_LD + kb) : Frag{};
                        acc = M::mma(cur.pf[kk], bf, acc);
                    }
                }
                const int j = jb + kTile * nn + l16;
                const int t0 = kTile * I + 4 * grp;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    T *dst = (t0 + r < len) ? og + (size_t(tok0 + t0 + r) * H + h) * DV + j : dummy;
                    __builtin_nontemporal_store(from_f32<T>(acc[r]), dst);
                }
            }
        }
    }

    // 3. S = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int item = wid + kWaves * i;
        if (item < NSI) {
            const int nn = item / NRT;
            floatx4 acc = S[i] * cur.d[i];
#pragma unroll
            for (int kk = 0; kk < Cfg::KSC; ++kk) {
                const int kb = kk * M::K + grp * M::KPL;
                const Frag bf = (kb < C) ? M::load(sUT + (kTile * nn + l16) * UT_LD + kb) : Frag{};
                acc = M::mma(cur.kt[i][kk], bf, acc);
            }
            S[i] = acc;
        }
    }
}

// Strided checkpoint: after the lc-th chunk of sequence n (0-based), when
// it is a full chunk and lc + 1 is a multiple of ck_every, the state goes to
// the sequence's checkpoint (lc + 1) / ck_every - 1.  The tests are uniform
// over the workgroup (scalar branches holding only stores).
template <class T, int DK, int DV, int C, int BV>
__device__ __forceinline__ void inter_ckpt(const PrefillArgs &a, const floatx4 (&S)[InterCfg<T, DK, DV, C, BV>::SPW],
                                           int n, int h, int lc, bool full, int wid, int grp, int l16, int jb) {
    using Cfg = InterCfg<T, DK, DV, C, BV>;
    if (!a.ckpt || !full || (lc + 1) % a.ck_every != 0) return;
    const int idx = (a.cu ? ld_const(a.ckoff, n) : n * a.ck_per_seq) + (lc + 1) / a.ck_every - 1;
    if (idx >= a.num_ckpt) return;
    float *dst = a.ckpt + (size_t(idx) * a.H + h) * DK * DV;
#pragma unroll
    for (int i = 0; i < Cfg::SPW; ++i) {
        const int item = wid + kWaves * i;
        if (item < Cfg::NSI) {
            const int m = item % Cfg::NRT, nn = item / Cfg::NRT;
#pragma unroll
            for (int r = 0; r < 4; ++r)  // non-temporal: read by no later step of this call
                __builtin_nontemporal_store(S[i][r], dst + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16);
        }
    }
}

template <class T, int DK, int DV, int C, int BV, int MODE>
__global__ __launch_bounds__(kThreads) void kda_inter_kernel(PrefillArgs a) {
    using Cfg = InterCfg<T, DK, DV, C, BV>;
    constexpr int NB = Cfg::NB, NRT = Cfg::NRT;
    constexpr int NSI = Cfg::NSI, SPW = Cfg::SPW, NS = Cfg::NS;
    constexpr int PT = 16 / sizeof(T);
    static_assert(MODE != kSumM || DV == DK, "a transition is dk x dk");
    __shared__ __align__(16) T sST[BV * (DK + PT)];
    __shared__ __align__(16) T sUT[BV * (C + PT)];

    const int H = a.H;
    const bool segmented = a.seg_len > 0;
    const int nseg = segmented ? a.nseg : 1;
    const int nchains = a.N * nseg * H;
    const int wg = blockIdx.x;
    int chain, blk;
    if ((nchains & 7) == 0) {
        // the NB blocks of one chain share an XCD (and its L2): workgroups
        // are dealt round-robin to the 8 XCDs by linear id
        const int xcd = wg & 7, slot = wg >> 3;
        blk = slot % NB;
        chain = xcd + 8 * (slot / NB);
    } else {
        chain = wg / NB;
        blk = wg - chain * NB;
    }
    // chain = (n * nseg + segment) * H + h
    const int h = chain % H, ns_idx = chain / H;
    const int n = ns_idx / nseg, sgi = ns_idx - n * nseg;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int grp = lane >> 4, l16 = lane & 15;
    const int jb = blk * BV;

    int c_begin, c_end, tok_start, tok_end, lc0 = 0;
    if (!a.cu) {
        c_begin = n * a.nc_seq;
        c_end = c_begin + a.nc_seq;
        tok_start = n * a.T;
        tok_end = tok_start + a.T;
        if (segmented) {
            lc0 = sgi * a.seg_len;  // chunks of the sequence before this segment
            c_begin += lc0;
            c_end = min(c_end, c_begin + a.seg_len);
            tok_start += lc0 * C;
            tok_end = min(tok_end, tok_start + a.seg_len * C);
        }
    } else {
        c_begin = min(a.coff[n], a.nc_max);
        c_end = min(max(a.coff[n + 1], c_begin), a.nc_max);
        tok_start = clampi(a.cu[n], 0, a.T);
        tok_end = clampi(a.cu[n + 1], tok_start, a.T);
    }

    // fp32 state tiles (m, nn): rows 16m.., value columns jb + 16nn..
    floatx4 S[SPW];
    const size_t sbase = size_t(chain) * DK * DV;
#pragma unroll
    for (int i = 0; i < SPW; ++i) {
        const int item = wid + kWaves * i;
        S[i] = zero4();
        if (item < NSI) {
            const int m = item % NRT, nn = item / NRT;
            if (MODE == kSumM) {
#pragma unroll
                for (int r = 0; r < 4; ++r) S[i][r] = (kTile * m + 4 * grp + r == jb + kTile * nn + l16) ? 1.f : 0.f;
            } else if (MODE == kFull && a.h0) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    S[i][r] = a.h0[sbase + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16];
            }
        }
    }
    // the initial state must have arrived before the first prefetch is
    // issued; otherwise every later wait on the loop header drains the ring
#pragma unroll
    for (int i = 0; i < SPW; ++i) asm volatile("" : "+v"(S[i]));

    T *og = static_cast<T *>(a.o);
    T *dummy = static_cast<T *>(a.dummy) + tid;
    InterStage<T, DK, DV, C, BV> st[NS];
    if (c_begin < c_end) {
#pragma unroll
        for (int s = 0; s < NS - 1; ++s)
            inter_load<T, DK, DV, C, BV, MODE>(st[s], a, min(c_begin + s, c_end - 1), h, wid, grp, l16, jb);
    }
    int gc = c_begin;
    // full groups of NS chunks, branch-free: the chunk loaded NS-1 steps
    // ahead is clamped to the last one (a harmless repeated load at the end)
    for (; gc + NS <= c_end; gc += NS) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            inter_load<T, DK, DV, C, BV, MODE>(st[(s + NS - 1) % NS], a, min(gc + s + NS - 1, c_end - 1), h, wid,
                                               grp, l16, jb);
            const int tok0 = tok_start + (gc + s - c_begin) * C;
            inter_chunk<T, DK, DV, C, BV, MODE>(st[s], S, sST, sUT, og, dummy, tok0, min(C, tok_end - tok0), H, h,
                                                wid, grp, l16, jb);
            if (MODE == kFull)
                inter_ckpt<T, DK, DV, C, BV>(a, S, n, h, lc0 + gc + s - c_begin, tok0 + C <= tok_end, wid, grp, l16,
                                             jb);
        }
    }
    // the last (c_end - gc) < NS chunks are already in st[0], st[1], ...
#pragma unroll
    for (int s = 0; s < NS - 1; ++s) {
        if (gc + s < c_end) {
            const int tok0 = tok_start + (gc + s - c_begin) * C;
            inter_chunk<T, DK, DV, C, BV, MODE>(st[s], S, sST, sUT, og, dummy, tok0, min(C, tok_end - tok0), H, h,
                                                wid, grp, l16, jb);
            if (MODE == kFull)
                inter_ckpt<T, DK, DV, C, BV>(a, S, n, h, lc0 + gc + s - c_begin, tok0 + C <= tok_end, wid, grp, l16,
                                             jb);
        }
    }

    // the end state: a segment summary (its own slot), or ht from the last
    // segment of the sequence (slot n * H + h)
    float *dst = nullptr;
    if (MODE != kFull) dst = a.ht + sbase;
    else if (a.ht && sgi == nseg - 1) dst = a.ht + size_t(n * H + h) * DK * DV;
    if (dst) {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT, nn = item / NRT;
#pragma unroll
                for (int r = 0; r < 4; ++r)  // non-temporal: read by no later step of this call
                __builtin_nontemporal_store(S[i][r], dst + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Kernel 2, loader-fed variant (bf16, 16-column value blocks, outputs).  The
// register-fed kernel above stalls for ~1,200 of its ~3,000 cycles per chunk
// issuing the next chunk's ~52 KiB of operand loads: every wave issues its
// share at once and the compute unit's vector-memory pipeline takes them at
// its own rate, while the products wait behind them in the same waves.  Here
// loader waves copy each chunk's operands (W, q e^Gam, K~^T, P, e^{Gam_last}
// and this block's Ut tiles, already in the order the products read them) into
// one of two LDS buffers two chunks ahead, and the four compute waves read
// them from LDS: their only global accesses are the o stores.  Both roles
// pass the same barriers: one before the chain, then the two of each chunk.
// Twelve loader waves: a compute unit issues 16-byte loads faster the more
// waves issue them (~41 B/clk from four waves, ~56 from sixteen), and with
// twelve each loader thread holds five units a stage, so the kernel fits 128
// VGPRs with no spill.  What bounds the chain is then the compute waves' own
// latency per chunk (S^T, X/O, state update and P U, two barriers).
// ---------------------------------------------------------------------------
constexpr int kWsLoaderWaves = 12;
template <int DK, int DV, int C, int NLW>
struct WsBuf {
    using M = Mma<bf16>;
    static constexpr int CP = kpad<bf16>(C);
    static constexpr int NT = C / kTile;
    // byte offsets inside one buffer
    static constexpr int oW = 0;
    static constexpr int oQ = oW + C * DK * 2;
    static constexpr int oK = oQ + C * DK * 2;
    static constexpr int oU = oK + DK * CP * 2;   // Ut tiles (I, this block), 256 values each
    static constexpr int oP = oU + NT * 256 * 2;  // P, lower-block operand order
    static constexpr int oD = oP + p_elems<bf16, C>() * 2;  // e^{Gam_last}, fp32
    static constexpr int bytes = oD + DK * 4;
    static constexpr int units = bytes / 16;       // 16-byte copy units, laid end to end as above
    static_assert(oQ % 16 == 0 && oK % 16 == 0 && oU % 16 == 0 && oP % 16 == 0 && oD % 16 == 0 && bytes % 16 == 0,
                  "16-byte units");
    static constexpr int kLoaders = kWave * NLW;   // loader threads
    static constexpr int UPT = (units + kLoaders - 1) / kLoaders;  // units per loader thread
    static constexpr size_t lds_bytes = size_t(2) * bytes;
};

// Copy unit lt + kLoaders * i of a chunk (clamped to the last unit, so the
// plan's addresses stay inside the chunk's regions).  Only the last step can
// run past the end; there the lanes whose unit does not exist neither load
// nor write (a clamped copy would have every such lane write the same 16
// bytes of LDS, and the youngest loader waves, which own those units, are
// the last to issue).
template <int DK, int DV, int C, int NLW, int i>
__device__ __forceinline__ int ws_unit(int lt) {
    using B = WsBuf<DK, DV, C, NLW>;
    return min(lt + B::kLoaders * i, B::units - 1);
}
template <int DK, int DV, int C, int NLW, int i>
__device__ __forceinline__ bool ws_live(int lt) {
    using B = WsBuf<DK, DV, C, NLW>;
    if constexpr (B::kLoaders * (i + 1) <= B::units) return true;
    else return lt + B::kLoaders * i < B::units;
}

// Where a loader thread's units come from.  The units run over W, q e^Gam,
// K~^T (contiguous spans of a chunk slot), this block's Ut tiles (512-byte
// spans: 32 units a tile), P and e^{Gam_last} (contiguous).  Every region
// starts at a multiple of 64 units and a loader wave's step i covers 64
// consecutive units, so the region of step i is uniform over the wave: its
// base and per-slot stride sit in scalar registers, and a lane keeps only
// its byte offset inside the slot's span, which is the same for every chunk.
template <int DK, int DV, int C, int NLW>
struct WsPlan {
    using B = WsBuf<DK, DV, C, NLW>;
    static constexpr int UW = C * DK * 2 / 16, UK = DK * B::CP * 2 / 16, UT = B::NT * 32;
    static constexpr int UP = p_elems<bf16, C>() * 2 / 16, UD = DK * 4 / 16;
    static constexpr int R1 = UW, R2 = 2 * UW, R3 = R2 + UK, R4 = R3 + UT, R5 = R4 + UP;
    static_assert(R1 % kWave == 0 && R2 % kWave == 0 && R3 % kWave == 0 && R4 % kWave == 0 && R5 % kWave == 0 &&
                      B::kLoaders % kWave == 0 && R5 + UD == B::units,
                  "regions of whole loader waves");
    typedef const __attribute__((address_space(1))) char gchar;  // global memory: vector-memory loads only
    const gchar *base[B::UPT];  // region base (uniform)
    unsigned stride[B::UPT];    // region bytes per chunk slot (uniform)
    unsigned voff[B::UPT];      // this lane's byte offset inside a slot's span

    template <int i>
    __device__ __forceinline__ void init_unit(const PrefillArgs &a, int lt, int nn0) {
        if constexpr (i < B::UPT) {
            const int u = ws_unit<DK, DV, C, NLW, i>(lt);
            const int u0 = __builtin_amdgcn_readfirstlane(u);
            const int r = (u0 >= R1) + (u0 >= R2) + (u0 >= R3) + (u0 >= R4) + (u0 >= R5);
            const void *bases[6] = {a.W, a.Qg, a.KtT, a.Ut, a.Ps, a.D};  // all in global memory
            constexpr unsigned strides[6] = {C * DK * 2, C * DK * 2, DK * B::CP * 2, C * DV * 2,
                                             p_elems<bf16, C>() * 2, DK * 4};
            constexpr int starts[6] = {0, R1, R2, R3, R4, R5};
            // (read back through readfirstlane: the values are uniform, and the
            // compiler then keeps them, and each slot's span base, in scalar
            // registers; the loads take the lane offset as a 32-bit VGPR)
            const unsigned long long b = reinterpret_cast<unsigned long long>(bases[r]);
            const unsigned lo = __builtin_amdgcn_readfirstlane(unsigned(b)),
                           hi = __builtin_amdgcn_readfirstlane(unsigned(b >> 32));
            base[i] = reinterpret_cast<const gchar *>((static_cast<unsigned long long>(hi) << 32) | lo);
            stride[i] = __builtin_amdgcn_readfirstlane(strides[r]);
            const int j = u - starts[r];
            voff[i] = r == 3 ? unsigned(((j / 32) * (DV / 16) + nn0) * 512 + (j % 32) * 16) : unsigned(j * 16);
            init_unit<i + 1>(a, lt, nn0);
        }
    }
    __device__ __forceinline__ u32x4 fetch(int i, size_t slot) const {
        const gchar *span = base[i] + slot * stride[i];
        return *reinterpret_cast<const __attribute__((address_space(1))) u32x4 *>(span + voff[i]);
    }
};

template <int DK, int DV, int C, int NLW, int i>
__device__ __forceinline__ void ws_fetch_unit(u32x4 *r, const WsPlan<DK, DV, C, NLW> &pl, size_t slot, int lt) {
    if constexpr (i < WsBuf<DK, DV, C, NLW>::UPT) {
        if (ws_live<DK, DV, C, NLW, i>(lt)) r[i] = pl.fetch(i, slot);
        ws_fetch_unit<DK, DV, C, NLW, i + 1>(r, pl, slot, lt);
    }
}

template <int DK, int DV, int C, int NLW, int i>
__device__ __forceinline__ void ws_put_unit(const u32x4 *r, unsigned char *dst, int lt) {
    if constexpr (i < WsBuf<DK, DV, C, NLW>::UPT) {
        if (ws_live<DK, DV, C, NLW, i>(lt)) *reinterpret_cast<u32x4 *>(dst + ws_unit<DK, DV, C, NLW, i>(lt) * 16) = r[i];
        ws_put_unit<DK, DV, C, NLW, i + 1>(r, dst, lt);
    }
}

// Units i .. iend - 1 of one staging step: unit i of a chunk already in
// registers (rp) goes to LDS, then unit i of a later chunk (slot) is
// requested into rf.  Alternating the two keeps the LDS and the
// vector-memory pipelines busy together.
template <int DK, int DV, int C, int NLW, int i, int iend>
__device__ __forceinline__ void ws_step(const u32x4 *rp, unsigned char *dst, u32x4 *rf,
                                        const WsPlan<DK, DV, C, NLW> &pl, size_t slot, int lt) {
    if constexpr (i < iend) {
        if (ws_live<DK, DV, C, NLW, i>(lt)) {
            *reinterpret_cast<u32x4 *>(dst + ws_unit<DK, DV, C, NLW, i>(lt) * 16) = rp[i];
            rf[i] = pl.fetch(i, slot);
        }
        ws_step<DK, DV, C, NLW, i + 1, iend>(rp, dst, rf, pl, slot, lt);
    }
}

template <int DK, int DV, int C, int NLW>
__global__ __launch_bounds__(kThreads + kWave * NLW) void kda_inter_ws_kernel(PrefillArgs a) {
    constexpr int BV = 16;
    using Cfg = InterCfg<bf16, DK, DV, C, BV>;
    using B = WsBuf<DK, DV, C, NLW>;
    using M = Mma<bf16>;
    constexpr int NRT = Cfg::NRT, NSI = Cfg::NSI, SPW = Cfg::SPW, XPW = Cfg::XPW;
    constexpr int NB = DV / BV;
    constexpr int PT = 8;
    static_assert(Cfg::NCT == 1 && XPW == 1 && C % M::K == 0,
                  "one 16-column tile per block, one output tile per wave, whole k-steps over the chunk");
    __shared__ __align__(16) bf16 sST[BV * (DK + PT)];
    __shared__ __align__(16) bf16 sUT[BV * (C + PT)];
    extern __shared__ __align__(16) unsigned char wsbuf[];

    const int H = a.H;
    const int nchains = (a.cu ? a.N : a.win_nn) * H;  // this launch's (sequence, head) chains
    const int wg = blockIdx.x;
    int chain, blk;
    if ((nchains & 7) == 0) {  // the NB blocks of a chain share an XCD
        const int xcd = wg & 7, slot = wg >> 3;
        blk = slot % NB;
        chain = xcd + 8 * (slot / NB);
    } else {
        chain = wg / NB;
        blk = wg - chain * NB;
    }
    const int h = chain % H, nw = chain / H, n = (a.cu ? 0 : a.win_n0) + nw;
    const int tid = threadIdx.x;
    const int wid_all = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int jb = blk * BV, nn0 = jb / kTile;

    int c_begin, c_end, tok_start, tok_end;
    if (!a.cu) {  // this launch's chunk window of the sequence
        c_begin = n * a.nc_seq + a.win_c0;
        c_end = c_begin + a.win_nc;
        tok_start = n * a.T + a.win_c0 * C;
        tok_end = n * a.T + a.T;
    } else {
        c_begin = min(a.coff[n], a.nc_max);
        c_end = min(max(a.coff[n + 1], c_begin), a.nc_max);
        tok_start = clampi(a.cu[n], 0, a.T);
        tok_end = clampi(a.cu[n + 1], tok_start, a.T);
    }
    const int nc = c_end - c_begin;  // chunks of this chain (may be 0)
    const int hc_begin = a.cu ? c_begin : nw * a.win_len;  // its first hand-off slot (intra_handoff)

    if (wid_all >= kWaves) {
        // ---------------- loader waves ----------------
        const int lt = tid - kThreads;
        constexpr int UPT = B::UPT;
        u32x4 st[3][UPT];
        WsPlan<DK, DV, C, NLW> pl;
        pl.template init_unit<0>(a, lt, nn0);
        auto fetch = [&](u32x4 (&r)[UPT], int c) {
            const size_t slot = size_t(hc_begin + min(c, nc - 1)) * H + h;
            ws_fetch_unit<DK, DV, C, NLW, 0>(r, pl, slot, lt);
        };
        auto put = [&](const u32x4 (&r)[UPT], int buf) { ws_put_unit<DK, DV, C, NLW, 0>(r, wsbuf + buf * B::bytes, lt); };
        // chunk x lives in register stage x % 3 and LDS buffer x & 1.  During
        // chunk c the loader writes chunk c + 2 into buffer c & 1 (read by the
        // compute waves at the top of chunk c, before the first barrier) and
        // requests chunk c + 4, half after each of the chunk's two barriers,
        // so neither half holds a barrier back.
        constexpr int HALF = UPT / 2;
        auto slot_of = [&](int x) { return size_t(hc_begin + min(x, nc - 1)) * H + h; };
        if (nc > 0) {
            fetch(st[0], 0);
            fetch(st[1], 1);
            fetch(st[2], 2);
            put(st[0], 0);
            put(st[1], 1);
            fetch(st[0], 3);
        }
        __syncthreads();  // chunks 0 and 1 staged
        int c = 0;
        for (; c + 3 <= nc; c += 3) {
#pragma unroll
            for (int s = 0; s < 3; ++s) {
                unsigned char *dst = wsbuf + ((c + s) & 1) * B::bytes;
                const size_t sl = slot_of(c + s + 4);
                __syncthreads();  // A
                ws_step<DK, DV, C, NLW, 0, HALF>(st[(s + 2) % 3], dst, st[(s + 1) % 3], pl, sl, lt);
                __syncthreads();  // B
                ws_step<DK, DV, C, NLW, HALF, UPT>(st[(s + 2) % 3], dst, st[(s + 1) % 3], pl, sl, lt);
            }
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            if (c + s < nc) {
                unsigned char *dst = wsbuf + ((c + s) & 1) * B::bytes;
                const size_t sl = slot_of(c + s + 4);
                __syncthreads();
                ws_step<DK, DV, C, NLW, 0, HALF>(st[(s + 2) % 3], dst, st[(s + 1) % 3], pl, sl, lt);
                __syncthreads();
                ws_step<DK, DV, C, NLW, HALF, UPT>(st[(s + 2) % 3], dst, st[(s + 1) % 3], pl, sl, lt);
            }
        }
        return;
    }

    // ---------------- compute waves ----------------
    const int wid = wid_all, lane = tid & 63;
    const int grp = lane >> 4, l16 = lane & 15;
    floatx4 S[SPW];
    const size_t sbase = (size_t(n) * H + h) * DK * DV;
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
    // Reads of a chunk's operands are split around the two barriers so that
    // none of them sits on the path S^T -> X/O -> S: W and q e^Gam of chunk
    // c + 1 (staged in buffer (c + 1) & 1 before barrier A of chunk c) are
    // read during chunk c's state update, and the rest of chunk c (Ut, K~^T,
    // P, e^{Gam_last}; rewritten by the loader only after barrier B) during
    // its X/O products.
    static_assert(B::UPT / 2 * B::kLoaders <= B::oK / 16,
                  "the loader's first half-step (after barrier A) rewrites only W and q e^Gam units");
    typedef M::Frag Frag;
    constexpr int ST_LD = DK + PT, UT_LD = C + PT;
    const int I = wid % Cfg::NT;
    const int t0 = kTile * I + 4 * grp;
    Frag w[Cfg::KSD], q[Cfg::KSD];
    auto read_wq = [&](const unsigned char *buf) {
#pragma unroll
        for (int kk = 0; kk < Cfg::KSD; ++kk) {
            const int off = ((I * Cfg::KSD + kk) * (16 * M::K) + lane * M::KPL) * 2;
            w[kk] = *reinterpret_cast<const bf16x8 *>(buf + B::oW + off);
            q[kk] = *reinterpret_cast<const bf16x8 *>(buf + B::oQ + off);
        }
    };
    // byte offset of this lane's first o value from its chunk's first row
    // (the next three are a row apart)
    const int ooff = (t0 * H * DV + jb + l16) * 2, orow = H * DV * 2;
    // S^T -> LDS in bf16, for the next chunk's products
    auto put_st = [&]() {
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT;
                store4(sST + l16 * ST_LD + kTile * m + 4 * grp, S[i][0], S[i][1], S[i][2], S[i][3]);
            }
        }
    };
    __syncthreads();  // chunks 0 and 1 staged
    if (nc > 0) read_wq(wsbuf);
    put_st();
    for (int c = 0; c < nc; ++c) {
        const unsigned char *buf = wsbuf + (c & 1) * B::bytes;
        const int tok0 = tok_start + c * C;
        const int len = max(0, min(C, tok_end - tok0));
        __syncthreads();  // A: S^T of this chunk's entering state is in LDS

        // 2. X = W S, O = (q e^Gam) S; U = Ut - X -> LDS.  The rest of this
        // chunk's operands are read alongside.
        floatx4 ax = zero4(), ao = zero4();
        Frag sf[Cfg::KSD];
#pragma unroll
        for (int kk = 0; kk < Cfg::KSD; ++kk) sf[kk] = M::load(sST + l16 * ST_LD + kk * M::K + grp * M::KPL);
        Quad<bf16> ut;
        ut.load(reinterpret_cast<const bf16 *>(buf + B::oU) + I * 256 + lane * 4);
        Frag pf[Cfg::KSC];  // rows of P of tile I; its k-blocks past the diagonal are zero
#pragma unroll
        for (int kk = 0; kk < Cfg::KSC; ++kk)
            pf[kk] = kk < p_nk<bf16>(I) ? *reinterpret_cast<const bf16x8 *>(
                                              buf + B::oP + ((p_pre<bf16>(I) + kk) * (16 * M::K) + lane * M::KPL) * 2)
                                        : bf16x8{};
        Frag kt[SPW][Cfg::KSC];
        floatx4 d[SPW];
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT;
#pragma unroll
                for (int kk = 0; kk < Cfg::KSC; ++kk)
                    kt[i][kk] = *reinterpret_cast<const bf16x8 *>(
                        buf + B::oK + ((m * Cfg::KSC + kk) * (16 * M::K) + lane * M::KPL) * 2);
                d[i] = *reinterpret_cast<const floatx4 *>(buf + B::oD + (kTile * m + 4 * grp) * 4);
            }
        }
#pragma unroll
        for (int kk = 0; kk < Cfg::KSD; ++kk) {
            ax = M::mma(w[kk], sf[kk], ax);
            ao = M::mma(q[kk], sf[kk], ao);
        }
        store4(sUT + l16 * UT_LD + t0, ut[0] - ax[0], ut[1] - ax[1], ut[2] - ax[2], ut[3] - ax[3]);
        __syncthreads();  // B

        // 3. S = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U, then its
        // S^T for the next chunk (this chunk's reads of S^T ended before
        // barrier B), then o = (q e^Gam) S + P U on the same U fragments,
        // off the path to the next chunk.  The next chunk's W, q e^Gam are
        // requested behind the U fragments (no branch: after the last chunk
        // the read is of a stale buffer, unused).
        Frag uf[Cfg::KSC];
#pragma unroll
        for (int kk = 0; kk < Cfg::KSC; ++kk) uf[kk] = M::load(sUT + l16 * UT_LD + kk * M::K + grp * M::KPL);
        read_wq(wsbuf + ((c + 1) & 1) * B::bytes);
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                floatx4 acc = S[i] * d[i];
#pragma unroll
                for (int kk = 0; kk < Cfg::KSC; ++kk) acc = M::mma(kt[i][kk], uf[kk], acc);
                S[i] = acc;
            }
        }
        put_st();
        __builtin_amdgcn_sched_barrier(0);  // keep P U behind the state's path
#pragma unroll
        for (int kk = 0; kk < Cfg::KSC; ++kk) ao = M::mma(pf[kk], uf[kk], ao);
        {
            // o rows of this chunk through a buffer resource whose range ends
            // at row len: stores of rows past the sequence's end are dropped.
            // The whole byte offset is the per-lane one, which the range check
            // covers (the range is uniform; readfirstlane keeps the resource
            // in scalar registers)
            const __amdgpu_buffer_rsrc_t orsrc = __builtin_amdgcn_make_buffer_rsrc(
                static_cast<bf16 *>(a.o) + (size_t(tok0) * H + h) * DV, (short)0,
                __builtin_amdgcn_readfirstlane(len * H * DV * 2), 0x00020000);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bf16 v = static_cast<bf16>(ao[r]);
                __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), orsrc, ooff + r * orow, 0, 0);
            }
        }
        inter_ckpt<bf16, DK, DV, C, BV>(a, S, n, h, a.win_c0 + c, tok0 + C <= tok_end, wid, grp, l16, jb);
    }
    if (a.ht) {
        float *dst = a.ht + size_t(n * H + h) * DK * DV;
#pragma unroll
        for (int i = 0; i < SPW; ++i) {
            const int item = wid + kWaves * i;
            if (item < NSI) {
                const int m = item % NRT, nn = item / NRT;
#pragma unroll
                for (int r = 0; r < 4; ++r)  // non-temporal: read by no later step of this call
                __builtin_nontemporal_store(S[i][r], dst + size_t(kTile * m + 4 * grp + r) * DV + jb + kTile * nn + l16);
            }
        }
    }
}

// Segment scan: the state entering segment j + 1 of (sequence n, head h) is
// Sin_{j+1} = M_j Sin_j + B_j, Sin_0 = h0 (or zero), in fp32, serially over
// the segments.  The serial steps are short when each thread owns little:
// one workgroup per (n, h, 8 value columns), each thread a 2 x 2 block of
// the dk x 8 tile, Sin_j staged in LDS.
template <int DK, int DV>
__global__ __launch_bounds__(256) void kda_seg_scan_kernel(PrefillArgs a) {
    constexpr int CB = 8;                       // columns per workgroup
    constexpr int NCB = DV / CB;
    constexpr int CQ = CB / 2;                  // 2-column groups
    constexpr int RQ = DK / 2;                  // 2-row groups
    static_assert(RQ * CQ <= 256 && DV % CB == 0, "scan tile");
    __shared__ __align__(16) float sS[DK][CB];
    const int H = a.H, nseg = a.nseg;
    const int wg = blockIdx.x, cb = wg % NCB, nh = wg / NCB;
    const int n = nh / H, h = nh - n * H;
    const int tid = threadIdx.x, cq = tid % CQ, rq = tid / CQ;
    const bool active = rq < RQ;
    const int c0 = cb * CB + 2 * cq;
    auto slot = [&](int j) { return size_t((n * nseg + j) * H + h); };
    for (int i = tid; i < DK * CB; i += 256) {
        const int r = i / CB, c = i - r * CB;
        const float x = a.h0 ? a.h0[size_t(n * H + h) * DK * DV + size_t(r) * DV + cb * CB + c] : 0.f;
        sS[r][c] = x;
        a.Sin[slot(0) * DK * DV + size_t(r) * DV + cb * CB + c] = x;
    }
    __syncthreads();
    for (int j = 0; j + 1 < nseg; ++j) {
        float acc[2][2];
        if (active) {
            const float *Mj = a.Mseg + slot(j) * DK * DK + size_t(2 * rq) * DK;
            const float *Bj = a.Bseg + slot(j) * DK * DV + size_t(2 * rq) * DV + c0;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const float2 b = *reinterpret_cast<const float2 *>(Bj + size_t(r) * DV);
                acc[r][0] = b.x;
                acc[r][1] = b.y;
            }
            for (int kk = 0; kk < DK; kk += 4) {
                const float4 m0 = *reinterpret_cast<const float4 *>(Mj + kk);
                const float4 m1 = *reinterpret_cast<const float4 *>(Mj + DK + kk);
                const float mv[2][4] = {{m0.x, m0.y, m0.z, m0.w}, {m1.x, m1.y, m1.z, m1.w}};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float2 s2 = *reinterpret_cast<const float2 *>(&sS[kk + q][2 * cq]);
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        acc[r][0] += mv[r][q] * s2.x;
                        acc[r][1] += mv[r][q] * s2.y;
                    }
                }
            }
        }
        __syncthreads();  // every read of Sin_j is done
        if (active) {
            float *dst = a.Sin + slot(j + 1) * DK * DV + size_t(2 * rq) * DV + c0;
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                *reinterpret_cast<float2 *>(&sS[2 * rq + r][2 * cq]) = make_float2(acc[r][0], acc[r][1]);
                *reinterpret_cast<float2 *>(dst + size_t(r) * DV) = make_float2(acc[r][0], acc[r][1]);
            }
        }
        __syncthreads();
    }
}

// Strided checkpoint from the accumulator-resident state (see inter_ckpt).
template <int DK, int DV>
__device__ __forceinline__ void chain_ckpt(const PrefillArgs &a, const floatx4 (&S)[DK / kTile], int n, int h, int lc,
                                           bool full, int grp, int l16, int nb) {
    if (!full || (lc + 1) % a.ck_every != 0) return;
    const int idx = (a.cu ? ld_const(a.ckoff, n) : n * a.ck_per_seq) + (lc + 1) / a.ck_every - 1;
    if (idx >= a.num_ckpt) return;
    float *dst = a.ckpt + (size_t(idx) * a.H + h) * DK * DV;
#pragma unroll
    for (int m = 0; m < DK / kTile; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[size_t(kTile * m + 4 * grp + r) * DV + nb + l16] = S[m][r];
}

// ---------------------------------------------------------------------------
// Kernel 2b (bf16): the state chain with the state held in MFMA accumulators.
// One workgroup per (chain, block of 16 * NWV value columns); wave w owns the
// 16 columns jb + 16 w of S, all dk rows, as 16x16 accumulator tiles (a lane
// holds rows 4 grp .. 4 grp + 3 of column l16 of each tile).  Products use
// the 16x16x32 bf16 MFMA with a permuted contraction order: slot j < 4 of a
// lane's 8 operand values is row 4 grp + j of tile 2p, slot j >= 4 row
// 4 grp + j - 4 of tile 2p + 1.  With that order the B operand of X = W S and
// O = (q e^Gam) S is just the lane's own accumulators of tiles 2p, 2p + 1,
// and U = Ut - X (token tiles 2q, 2q + 1) is the B operand of both
// S += K~^T U and o = O + P U: the state and U never leave the wave.  The A
// operands every wave needs — W, q e^Gam, K~^T, P — are staged per chunk in
// LDS in the same permuted order (one 16-byte read per operand), with
// e^{Gam_last}, double-buffered, from a ring of NS register stages loaded
// NS - 1 chunks ahead; one barrier per chunk (the d = 128 output chains: one
// buffer, two barriers, see ONE).  The loop runs whole NS-chunk groups;
// chunks past the chain's end are inactive (state kept, nothing stored):
// branch-free, static ring indices.
// ---------------------------------------------------------------------------
template <int DK, int DV, int C, int NWV, int MODE>
struct ChainCfg {
    static constexpr int NTHR = kWave * NWV * (MODE == kSumBM ? 2 : 1);
    static constexpr int BW = kTile * NWV;                  // columns per workgroup (per half in kSumBM)
    static constexpr int NT = C / kTile, MT = DK / kTile;
    static constexpr int NQ = (NT + 1) / 2, MP = MT / 2;    // 32-wide token / dk slices
    static constexpr int CP = kpad<bf16>(C);                // K~^T row length (operand order)
    static constexpr bool HAS_Q = MODE == kFull;           // q e^Gam and P: outputs
    static constexpr int W_EL = C * DK, K_EL = DK * CP;     // bf16 elements per chunk
    static constexpr int PW = W_EL * 2 / 16, PK = K_EL * 2 / 16, PD = DK * 4 / 16;  // 16-byte pieces
    static constexpr int PP = HAS_Q ? p_elems<bf16, C>() * 2 / 16 : 0;
    static constexpr int KB = PW * (HAS_Q ? 2 : 1);        // first K~^T piece
    static constexpr int PB = KB + PK;                      // first P piece
    static constexpr int DB = PB + PP;                      // first e^{Gam_last} piece
    static constexpr int P = DB + PD;
    static_assert(PW % 64 == 0 && PK % 64 == 0 && PP % 64 == 0, "whole 1 KiB operand blocks");
    static constexpr int PPT = (P + NTHR - 1) / NTHR;       // pieces per thread
    static constexpr int BUF = PPT * NTHR * 16;             // bytes per LDS buffer (padded)
    // d = 128 output chains: one LDS buffer and two register stages, so that
    // two workgroups share a compute unit (the chain is latency-bound at one
    // wave per SIMD); the buffer is rewritten between two barriers
    static constexpr bool ONE = MODE == kFull && DK == 128 && DV == 128 && C == 64 && NWV == 4;
    static constexpr int NBUF = ONE ? 1 : 2;
    static constexpr int NS = ONE || PPT > 16 ? 2 : 4;      // register stages (fewer when each holds more)
    static_assert(NS % 2 == 0, "the LDS buffer of a chunk is its index mod 2");
    static_assert(DK % 32 == 0 && NTHR % kWave == 0, "chain shapes");
};

template <int DK, int DV, int C, int NWV, int MODE>
struct ChainStage {
    using Cfg = ChainCfg<DK, DV, C, NWV, MODE>;
    u32x4 stg[Cfg::PPT];                  // this thread's pieces of the staged operands
    bf16x4 ut[Cfg::NT];                   // Ut at this lane's positions of its column block
};

// Loads one chunk's stage: 16-byte pieces p = tid + NTHR i of the operand-
// order W, q e^Gam, K~^T, of P (lower-block order) and of e^{Gam_last}, laid
// end to end; Ut (quad order) at this lane's positions.  Bases are uniform
// (scalar registers).
template <int DK, int DV, int C, int NWV, int MODE>
__device__ __forceinline__ void chain_load(ChainStage<DK, DV, C, NWV, MODE> &st, const PrefillArgs &a, int gc, int h,
                                           int tid, int loff, int nblk, bool isM) {
    using Cfg = ChainCfg<DK, DV, C, NWV, MODE>;
    const size_t slot = size_t(gc) * a.H + h;
    const char *W = static_cast<const char *>(a.W) + slot * Cfg::W_EL * 2;
    const char *Q = static_cast<const char *>(a.Qg) + slot * Cfg::W_EL * 2;
    const char *K = static_cast<const char *>(a.KtT) + slot * Cfg::K_EL * 2;
    const char *Ps = static_cast<const char *>(a.Ps) + slot * p_elems<bf16, C>() * 2;
    const char *D = reinterpret_cast<const char *>(a.D + slot * DK);
#pragma unroll
    for (int i = 0; i < Cfg::PPT; ++i) {
        const int p = min(tid + Cfg::NTHR * i, Cfg::P - 1);  // the padding re-reads the last piece
        const char *src;
        if (p < Cfg::PW) src = W + p * 16;
        else if (Cfg::HAS_Q && p < Cfg::KB) src = Q + (p - Cfg::PW) * 16;
        else if (p < Cfg::PB) src = K + (p - Cfg::KB) * 16;
        else if (Cfg::HAS_Q && p < Cfg::DB) src = Ps + (p - Cfg::PB) * 16;
        else src = D + (p - Cfg::DB) * 16;
        st.stg[i] = *reinterpret_cast<const u32x4 *>(src);
    }
    if (MODE != kSumM && !(MODE == kSumBM && isM)) {
        // quad order: tile (I, nblk) is 256 values, lane l holds 4 of them
        const char *U = reinterpret_cast<const char *>(static_cast<const bf16 *>(a.Ut) + slot * C * DV + nblk * 256);
#pragma unroll
        for (int I = 0; I < Cfg::NT; ++I) st.ut[I] = *reinterpret_cast<const bf16x4 *>(U + I * (DV / kTile) * 512 + loff);
    }
}

// Writes the stage into one LDS buffer.  A 16-byte operand-order piece (lane
// ln = l16 + 16 q of its block: 8 consecutive k from 8 q) goes, as two
// 8-byte halves, to the permuted order: the half with k offset c = 8 q + 4 h
// lands in lane l16 + 16 g of the same block, slot c / 16, with g = (c % 16)
// / 4.  K~^T and P columns past the chunk (the pad of a 16-token chunk)
// become 0.
template <int DK, int DV, int C, int NWV, int MODE>
__device__ __forceinline__ void chain_stage_write(unsigned char *buf, const ChainStage<DK, DV, C, NWV, MODE> &st,
                                                  int tid) {
    using Cfg = ChainCfg<DK, DV, C, NWV, MODE>;
#pragma unroll
    for (int i = 0; i < Cfg::PPT; ++i) {
        const int p = tid + Cfg::NTHR * i;
        const u32x4 v = st.stg[i];
        if (p >= Cfg::DB) {  // e^{Gam_last} and the padding: as is
            *reinterpret_cast<u32x4 *>(buf + p * 16) = v;
            continue;
        }
        const int blk = p >> 6, ln = p & 63, l16 = ln & 15, q = ln >> 4;
        const int s0 = q >> 1;                                      // slot of both halves
        const int g0 = 2 * (q & 1);                                 // lane group of half 0; half 1: g0 + 1
        u32x2 lo{v[0], v[1]}, hi{v[2], v[3]};
        if (C < 32 && p >= Cfg::KB && s0 == 1) lo = hi = u32x2{0u, 0u};  // K~^T, P pad columns
        unsigned char *base = buf + blk * 1024 + l16 * 16 + 8 * s0;
        *reinterpret_cast<u32x2 *>(base + (16 * g0) * 16) = lo;
        *reinterpret_cast<u32x2 *>(base + (16 * (g0 + 1)) * 16) = hi;
    }
}

template <int DK, int DV, int C, int NWV, int MODE>
__global__ __launch_bounds__(kWave * NWV * (MODE == kSumBM ? 2 : 1), (ChainCfg<DK, DV, C, NWV, MODE>::ONE ? 2 : 1))
void kda_chain_kernel(PrefillArgs a) {
    using Cfg = ChainCfg<DK, DV, C, NWV, MODE>;
    using Stage = ChainStage<DK, DV, C, NWV, MODE>;
    using M = Mma<bf16>;
    constexpr int NT = Cfg::NT, MT = Cfg::MT, NQ = Cfg::NQ, MP = Cfg::MP, NS = Cfg::NS, NB = DV / Cfg::BW;
    constexpr bool ONE = Cfg::ONE;
    static_assert((MODE != kSumM && MODE != kSumBM) || DV == DK, "a transition is dk x dk");
    static_assert(DV % Cfg::BW == 0, "chain blocks");
    __shared__ __align__(16) unsigned char sbuf[Cfg::NBUF][Cfg::BUF];

    const int H = a.H;
    const bool segmented = a.seg_len > 0;
    const int nseg = segmented ? a.nseg : 1;
    const int nchains = a.N * nseg * H;
    const int wg = blockIdx.x;
    int chain, blk;
    if ((nchains & 7) == 0) {  // the NB blocks of a chain share an XCD (and its L2)
        const int xcd = wg & 7, sl = wg >> 3;
        blk = sl % NB;
        chain = xcd + 8 * (sl / NB);
    } else {
        chain = wg / NB;
        blk = wg - chain * NB;
    }
    const int h = chain % H, ns_idx = chain / H;
    const int n = ns_idx / nseg, sgi = ns_idx - n * nseg;
    if (MODE != kFull && sgi == nseg - 1) return;  // the scan never reads the last segment's summary
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: column bases stay scalar
    const int grp = lane >> 4, l16 = lane & 15;
    // the transition's waves (all of them in kSumM, the second half in kSumBM)
    const bool isM = MODE == kSumM || (MODE == kSumBM && wid >= NWV);
    const int nb = blk * Cfg::BW + kTile * (MODE == kSumBM && isM ? wid - NWV : wid);  // first column
    const int nblk = nb / kTile;

    int c_begin, c_end, tok_start, tok_end, lc0 = 0;
    if (!a.cu) {
        c_begin = n * a.nc_seq;
        c_end = c_begin + a.nc_seq;
        tok_start = n * a.T;
        tok_end = tok_start + a.T;
        if (segmented) {
            lc0 = sgi * a.seg_len;
            c_begin += lc0;
            c_end = min(c_end, c_begin + a.seg_len);
            tok_start += lc0 * C;
            tok_end = min(tok_end, tok_start + a.seg_len * C);
        }
    } else {
        c_begin = min(ld_const(a.coff, n), a.nc_max);
        c_end = min(max(ld_const(a.coff, n + 1), c_begin), a.nc_max);
        tok_start = clampi(ld_const(a.cu, n), 0, a.T);
        tok_end = clampi(ld_const(a.cu, n + 1), tok_start, a.T);
    }

    // S tile m: rows 16 m + 4 grp + r, column nb + l16
    floatx4 S[MT];
    const size_t sbase = size_t(chain) * DK * DV;
#pragma unroll
    for (int m = 0; m < MT; ++m) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = kTile * m + 4 * grp + r, col = nb + l16;
            float x = 0.f;
            if (isM) x = (row == col) ? 1.f : 0.f;
            else if (MODE == kFull && a.h0) x = a.h0[sbase + size_t(row) * DV + col];
            S[m][r] = x;
        }
    }
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(S[m]));

    static_assert(Cfg::BUF <= 65536 - 64 * MT, "staged offsets fit the LDS immediate field");
    const int nchunks = c_end - c_begin;
    const int last = c_end - 1;
    const int loff = 8 * lane;
    Stage st[NS];
    if (nchunks > 0) {
#pragma unroll
        for (int s = 0; s < NS; ++s)
            chain_load<DK, DV, C, NWV, MODE>(st[s], a, min(c_begin + s, last), h, tid, loff, nblk, isM);
        chain_stage_write<DK, DV, C, NWV, MODE>(sbuf[0] + opaque(0), st[0], tid);
    }
    __syncthreads();

    const int groups = (nchunks + NS - 1) / NS;
    for (int gi = 0; gi < groups; ++gi) {
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int k = gi * NS + s;           // chunk index within the chain
            const int c = c_begin + k;
            const bool active = k < nchunks;
            // stage chunk c + 1 into the other buffer (opaque per-chunk bases
            // keep the compiler from holding every LDS address in a register)
            if (!ONE)
                chain_stage_write<DK, DV, C, NWV, MODE>(sbuf[0] + opaque(((s + 1) & 1) * Cfg::BUF), st[(s + 1) % NS],
                                                        tid);
            const int bsel = ONE ? 0 : (s & 1);
            const unsigned char *ra = sbuf[0] + opaque(bsel * Cfg::BUF + 16 * lane);
            const unsigned char *rd = sbuf[0] + opaque(bsel * Cfg::BUF + Cfg::DB * 16 + 16 * grp);
            const Stage &cur = st[s];

            // B operands from the state: tiles 2p, 2p + 1
            M::Frag sb[MP];
#pragma unroll
            for (int pp = 0; pp < MP; ++pp)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    sb[pp][j] = static_cast<bf16>(S[2 * pp][j]);
                    sb[pp][4 + j] = static_cast<bf16>(S[2 * pp + 1][j]);
                }
            const int tok0 = tok_start + k * C;
            const int len = active ? min(C, tok_end - tok0) : 0;
            // o rows of this chunk through a buffer resource whose range ends
            // at row len: stores of rows past the sequence's end are dropped.
            // The whole byte offset goes in the per-lane (VGPR) offset: the
            // range check of a raw buffer access covers that offset only, not
            // the scalar one.
            __amdgpu_buffer_rsrc_t orsrc;
            if (MODE == kFull)
                orsrc = __builtin_amdgcn_make_buffer_rsrc(static_cast<bf16 *>(a.o) + (size_t(tok0) * H + h) * DV + nb,
                                                          (short)0, len * H * DV * 2, 0x00020000);
            M::Frag ub[NQ];
#pragma unroll
            for (int qq = 0; qq < NQ; ++qq) ub[qq] = M::Frag{};
            floatx4 oacc[NT];
#pragma unroll
            for (int I = 0; I < NT; ++I) {
                floatx4 xa = zero4(), oa = zero4();
#pragma unroll
                for (int pp = 0; pp < MP; ++pp) {
                    const int blkoff = (I * MP + pp) * 1024;
                    xa = M::mma(*reinterpret_cast<const M::Frag *>(ra + blkoff), sb[pp], xa);
                    if (Cfg::HAS_Q) oa = M::mma(*reinterpret_cast<const M::Frag *>(ra + Cfg::PW * 16 + blkoff), sb[pp], oa);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    ub[I >> 1][4 * (I & 1) + r] =
                        static_cast<bf16>((isM ? 0.f : static_cast<float>(cur.ut[I][r])) - xa[r]);
                oacc[I] = oa;
            }
            if (MODE == kFull) {
                // o = (q e^Gam) S + P U: P's kept k-blocks of row tile I, in
                // the same permuted order as U
#pragma unroll
                for (int I = 0; I < NT; ++I) {
                    floatx4 acc = oacc[I];
#pragma unroll
                    for (int qq = 0; qq < p_nk<bf16>(I); ++qq)
                        acc = M::mma(*reinterpret_cast<const M::Frag *>(ra + Cfg::PB * 16 + (p_pre<bf16>(I) + qq) * 1024),
                                     ub[qq], acc);
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const bf16 v = static_cast<bf16>(acc[r]);
                        __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(unsigned short, v), orsrc,
                                                              ((kTile * I + 4 * grp + r) * H * DV + l16) * 2, 0, 0);
                    }
                }
            }
            // S = Diag(e^{Gam_last}) S + (k e^{Gam_last - Gam})^T U  (kept as is past the end)
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const float4 d = *reinterpret_cast<const float4 *>(rd + 64 * m);
                floatx4 acc = S[m] * floatx4{d.x, d.y, d.z, d.w};
#pragma unroll
                for (int qq = 0; qq < NQ; ++qq)
                    acc = M::mma(*reinterpret_cast<const M::Frag *>(ra + Cfg::KB * 16 + (m * (Cfg::CP / 32) + qq) * 1024),
                                 ub[qq], acc);
                S[m] = active ? acc : S[m];
            }
            if (MODE == kFull && active && a.ckpt)
                chain_ckpt<DK, DV>(a, S, n, h, lc0 + k, tok0 + C <= tok_end, grp, l16, nb);
            // this stage's registers now take chunk c + NS
            chain_load<DK, DV, C, NWV, MODE>(st[s], a, min(c + NS, last), h, tid, loff, nblk, isM);
            __syncthreads();
            if (ONE) {  // every read of chunk c is done: the buffer takes chunk c + 1
                chain_stage_write<DK, DV, C, NWV, MODE>(sbuf[0] + opaque(0), st[(s + 1) % NS], tid);
                __syncthreads();
            }
        }
    }

    float *dst = nullptr;
    if (MODE == kSumBM) dst = (isM ? a.Mseg : a.Bseg) + sbase;
    else if (MODE != kFull) dst = a.ht + sbase;
    else if (a.ht && sgi == nseg - 1) dst = a.ht + size_t(n * H + h) * DK * DV;
    if (dst) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[size_t(kTile * m + 4 * grp + r) * DV + nb + l16] = S[m][r];
    }
}

// Loader-fed state chain over this launch's chunks (bf16, 16-column blocks).
template <int DK, int DV, int C>
hipError_t launch_ws_chain(const PrefillArgs &a, hipStream_t s) {
    constexpr int NLW = kWsLoaderWaves;
    using WB = WsBuf<DK, DV, C, NLW>;
    hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&kda_inter_ws_kernel<DK, DV, C, NLW>),
                                      int(WB::lds_bytes));
    if (e != hipSuccess) return e;
    const int nwg = (a.cu ? a.N : a.win_nn) * a.H * (DV / 16);
    if (nwg > 0) {
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_ws_kernel<DK, DV, C, NLW>), dim3(nwg), dim3(kThreads + kWave * NLW),
                           WB::lds_bytes, s, a);
        prof_end(s, "kda_inter");
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Host-side launch of one (dtype, dk, dv, chunk, bv) instance.
// ---------------------------------------------------------------------------
template <class T, int DK, int DV, int C, int BV>
hipError_t launch_prefill_instance(const PrefillArgs &a, hipStream_t s) {
    using Ly = IntraLds<T, DK, DV, C>;
    static_assert(Ly::bytes <= 160 * 1024, "intra-chunk LDS exceeds 160 KiB");
    {
        hipError_t e = ensure_dynamic_lds(reinterpret_cast<const void *>(&kda_intra_kernel<T, DK, DV, C>), int(Ly::bytes));
        if (e != hipSuccess) return e;
    }
    // persistent: one workgroup per compute unit (LDS allows one), each
    // walking (chunk, head) items with its next item's inputs in flight
    auto launch_intra = [&](const PrefillArgs &b) -> hipError_t {
        const int items = intra_groups(b) * b.H;
        if (b.nc_max <= 0 || items <= 0) return hipSuccess;
        const int grid = items < b.num_cu ? items : b.num_cu;
        prof_begin(s);
        hipLaunchKernelGGL((kda_intra_kernel<T, DK, DV, C>), dim3(grid), dim3(kIThreads), Ly::bytes, s, b);
        prof_end(s, "kda_intra");
        return hipGetLastError();
    };
    if (a.nwin > 1) {
        // windows: each window's intra-chunk pass, then its state pass
        // (loader-fed chain, fixed-length batches): groups of win_grp
        // sequences, and for each group its chunk windows, the state carried
        // from one to the next
        if constexpr (sizeof(T) == 2 && DK == 128 && DV == 128 && C == 64 && BV == 16) {
            if (a.cu || a.seg_len > 0 || a.win_len <= 0 || a.win_grp <= 0) return hipErrorInvalidValue;
            for (int n0 = 0; n0 < a.N; n0 += a.win_grp) {
                for (int c0 = 0; c0 < a.nc_seq; c0 += a.win_len) {
                    PrefillArgs b = a;
                    b.win_n0 = n0;
                    b.win_nn = min(a.win_grp, a.N - n0);
                    b.fd_win_nn = make_fastdiv(uint32_t(b.win_nn));
                    b.win_c0 = c0;
                    b.win_nc = min(a.win_len, a.nc_seq - c0);
                    if (c0 > 0) b.h0 = a.carry;
                    if (c0 + b.win_nc < a.nc_seq) b.ht = a.carry;
                    hipError_t e = launch_intra(b);
                    if (e == hipSuccess) e = launch_ws_chain<DK, DV, C>(b, s);
                    if (e != hipSuccess) return e;
                }
            }
            return hipSuccess;
        } else {
            return hipErrorInvalidValue;
        }
    }
    {
        hipError_t e = launch_intra(a);
        if (e != hipSuccess) return e;
    }
    if constexpr (sizeof(T) == 2) {
        if (a.seg_len > 0) {
            // bf16 segments: the accumulator-resident chain, 16 * NWV columns
            // per workgroup (fewer copies of the shared operands, which is
            // what bounds the many-chain segment passes).  One chain per
            // (sequence, head) keeps the register-operand kernel below, whose
            // shorter per-chunk latency wins when there are few chains.
            constexpr int NWV = DV / kTile < 4 ? DV / kTile : 4, NWK = DK / kTile < 4 ? DK / kTile : 4;
            constexpr int BWV = kTile * NWV, BWK = kTile * NWK;
            const int nsc = a.N * a.nseg * a.H;
            PrefillArgs b = a;
            b.h0 = nullptr;
            b.ht = a.Bseg;
            b.ckpt = nullptr;
            if constexpr (DK == DV) {
                // both summaries in one pass over the chunk operands
                prof_begin(s);
                hipLaunchKernelGGL((kda_chain_kernel<DK, DV, C, NWV, kSumBM>), dim3(nsc * (DV / BWV)),
                                   dim3(2 * kWave * NWV), 0, s, b);
                prof_end(s, "kda_seg_sum_bm");
            } else {
                prof_begin(s);
                hipLaunchKernelGGL((kda_chain_kernel<DK, DV, C, NWV, kSumB>), dim3(nsc * (DV / BWV)),
                                   dim3(kWave * NWV), 0, s, b);
                prof_end(s, "kda_seg_sum_b");
                PrefillArgs m = b;
                m.ht = a.Mseg;
                prof_begin(s);
                hipLaunchKernelGGL((kda_chain_kernel<DK, DK, C, NWK, kSumM>), dim3(nsc * (DK / BWK)),
                                   dim3(kWave * NWK), 0, s, m);
                prof_end(s, "kda_seg_sum_m");
            }
            prof_begin(s);
            hipLaunchKernelGGL((kda_seg_scan_kernel<DK, DV>), dim3(a.N * a.H * (DV / 8)), dim3(256), 0, s, a);
            prof_end(s, "kda_seg_scan");
            PrefillArgs f = a;
            f.h0 = a.Sin;
            prof_begin(s);
            hipLaunchKernelGGL((kda_chain_kernel<DK, DV, C, NWV, kFull>), dim3(nsc * (DV / BWV)), dim3(kWave * NWV), 0,
                               s, f);
            prof_end(s, "kda_inter");
            return hipGetLastError();
        }
    }
    if (a.seg_len > 0) {
        // segment-parallel chain: summaries, scan, then the output chains
        constexpr int SB = 32;  // value-column block of the segmented chains
        static_assert(DV % SB == 0 && DK % SB == 0, "segment blocks");
        const int nsc = a.N * a.nseg * a.H;
        PrefillArgs b = a;
        b.h0 = nullptr;
        b.ht = a.Bseg;
        b.ckpt = nullptr;
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, DV, C, SB, kSumB>), dim3(nsc * (DV / SB)), dim3(kThreads), 0, s,
                           b);
        prof_end(s, "kda_seg_sum_b");
        PrefillArgs m = b;
        m.ht = a.Mseg;
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, DK, C, SB, kSumM>), dim3(nsc * (DK / SB)), dim3(kThreads), 0, s,
                           m);
        prof_end(s, "kda_seg_sum_m");
        prof_begin(s);
        hipLaunchKernelGGL((kda_seg_scan_kernel<DK, DV>), dim3(a.N * a.H * (DV / 8)), dim3(256), 0, s, a);
        prof_end(s, "kda_seg_scan");
        PrefillArgs f = a;
        f.h0 = a.Sin;
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, DV, C, SB, kFull>), dim3(nsc * (DV / SB)), dim3(kThreads), 0, s,
                           f);
        prof_end(s, "kda_inter");
        return hipGetLastError();
    }
    const int nwg = a.N * a.H * (DV / BV);
    if constexpr (sizeof(T) == 2 && DK == 128 && DV == 128 && C == 64 && BV == 16) {
        // loader-fed state chain (one chain per (sequence, head), no segments)
        return launch_ws_chain<DK, DV, C>(a, s);
    }
    if (nwg > 0) {
        prof_begin(s);
        hipLaunchKernelGGL((kda_inter_kernel<T, DK, DV, C, BV, kFull>), dim3(nwg), dim3(kThreads), 0, s, a);
        prof_end(s, "kda_inter");
    }
    return hipGetLastError();
}

}  // namespace kda
