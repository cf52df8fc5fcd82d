// Internal interface between the C ABI (kda_api.cpp) and the kernel
// translation units.  Not installed; no torch or Python types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

// Division by a divisor fixed for a launch, as a multiply-high and two
// shifts (Granlund and Montgomery, "Division by Invariant Integers using
// Multiplication", PLDI 1994, the round-up method for unsigned operands):
// with l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, the quotient
// of any 32-bit n is (t + ((n - t) >> min(l, 1))) >> max(l - 1, 0), where
// t = mulhi(m, n).  Built on the host; a zero divisor is taken as 1.
struct FastDiv {
    uint32_t m;
    uint32_t s1, s2;
};
inline FastDiv make_fastdiv(uint32_t d) {
    if (d == 0) d = 1;
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    FastDiv f;
    f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
    f.s1 = l < 1 ? l : 1;
    f.s2 = l > 1 ? l - 1 : 0;
    return f;
}
// n / d for a non-negative n (on the device, uniform operands stay scalar:
// the high half of the 64-bit product is one s_mul_hi_u32)
__host__ __device__ inline int fdiv(int n, const FastDiv &f) {
    const uint32_t un = uint32_t(n), t = uint32_t((uint64_t(f.m) * un) >> 32);
    return int((t + ((un - t) >> f.s1)) >> f.s2);
}

// Everything the prefill kernels need, by value.
struct PrefillArgs {
    const void *q, *k, *v;     // [rows][H][dk|dv] in the compute dtype
    const float *g, *beta;     // [rows][H][dk], [rows][H]
    const float *h0;           // [N][H][dk][dv] or null
    const int32_t *cu;         // packed sequence offsets [N+1] or null
    int32_t *coff;             // per-sequence first chunk slot [N+1] (packed only)
    int T;                     // tokens per sequence (fixed) or in total (packed)
    int H, N;
    int nc_max;                // chunk slots in the workspace
    int nc_seq;                // chunks per sequence (fixed-length batches)
    int num_cu;                // compute units of the device (persistent grids)
    void *o;                   // [rows][H][dv]
    float *ht;                 // [N][H][dk][dv] or null
    // workspace, per (chunk slot, head); "operand" / "quad" order are the
    // wave-read orders defined in kda_prefill_impl.h:
    void *W;                   // [C][dk]  (I+A)^-1 (beta k e^Gam), operand order
    void *Qg;                  // [C][dk]  q e^Gam, operand order
    void *KtT;                 // [dk][Cp] (k e^{Gam_last - Gam})^T, operand order
    void *Ut;                  // [C][dv]  (I+A)^-1 (beta v), quad order
    void *Ps;                  // [C][C]   scores P (lower by 16-token tiles), lower-block operand order
    float *D;                  // [dk]     e^{Gam_last}
    void *dummy;               // 1 KiB sink for the o rows past a sequence's end
    // strided state checkpoints (null ckpt: none): after every ck_every
    // chunks of a sequence (a full chunk ending there), S goes to checkpoint
    // ckoff[n] + j (packed) or n * ck_per_seq + j (fixed length) of
    // ckpt [num_ckpt][H][dk][dv]; indices at or past num_ckpt are dropped
    float *ckpt;
    int32_t *ckoff;            // per-sequence first checkpoint [N+1] (packed only)
    int ck_every, ck_per_seq, num_ckpt;
    // segment-parallel state chain (fixed-length batches only; seg_len 0:
    // off).  Sequence n's chunks split into nseg segments of seg_len chunks;
    // segment chain (n * nseg + j) * H + h.  Mseg [chains][dk][dk] and Bseg
    // [chains][dk][dv]: the segment's transition and zero-start end state;
    // Sin [chains][dk][dv]: the true state entering each segment.
    int seg_len, nseg;
    float *Mseg, *Bseg, *Sin;
    // windows (fixed-length batches on the loader-fed chain only): the call
    // runs as (intra-chunk pass, state pass) pairs, one per window: groups of
    // win_grp sequences, and inside each group chunk windows
    // [w win_len, min((w + 1) win_len, nc_seq)) (several only when
    // win_grp = 1), the state handed from one chunk window to the next
    // through carry [N][H][dk][dv].  A launch covers sequences
    // [win_n0, win_n0 + win_nn) and their chunks [win_c0, win_c0 + win_nc)
    // (0, N, 0, nc_seq: all).  nwin: the number of windows (1: none).
    int nwin, win_grp, win_len, win_n0, win_nn, win_c0, win_nc;
    float *carry;
    // the divisions of the intra-chunk pass's item walk: by H, by nc_seq and
    // by win_nn (set right before each launch)
    FastDiv fd_H, fd_nc_seq, fd_win_nn;
};

// Segment plan of a prefill: segments when long fixed-length sequences have
// too few (sequence, head) chains to occupy the device.  A pure function of
// the sizes, so the workspace size query and the call agree.
struct SegPlan {
    int nseg, seg_len;  // nseg 1, seg_len 0: no segmentation
};
SegPlan seg_plan(bool packed, int dtype, int dk, int dv, int C, int N, int H, int nc_seq);

// Windows of a prefill: win_grp sequences per window and chunk windows per
// sequence (nchunk > 1 only with win_grp = 1); {N, 1}: none.  A pure
// function of the sizes, like the segment plan, so the workspace size query
// and the call agree.
struct WinPlan {
    int grp, nchunk;
};
WinPlan win_plan(bool packed, int dtype, int dk, int dv, int C, int N, int H, int nc_seq, int nseg);

// Workspace carve-up shared by the size query and the prefill call.
struct PrefillLayout {
    size_t coff, ckoff, W, Qg, KtT, Ut, Ps, D, Mseg, Bseg, Sin, carry, dummy, flag, total;
};
PrefillLayout prefill_layout(int nc_max, int H, int N, int dk, int dv, int C,
                             size_t elem_bytes, int nseg, int nwin);
// bytes of one (chunk, head) slot of the hand-off from the intra-chunk pass
// to the state pass (W, q e^Gam, K~^T, Ut, P, e^{Gam_last})
size_t handoff_slot_bytes(int dk, int dv, int C, size_t elem_bytes);
// chunk length rounded up to the MFMA contraction of the dtype (K~^T pad)
inline int chunk_pad(int C, size_t elem_bytes) {
    const int k = elem_bytes == 2 ? 32 : 4;
    return (C + k - 1) / k * k;
}

// Elements of a chunk's score matrix P in lower-block operand order: row
// tile I (16 tokens) keeps only the k-blocks (16 x kstep values, kstep the
// MFMA contraction: 32 for bf16, 4 for fp32) that reach its diagonal, i.e.
// ceil(16 (I + 1) / kstep) of them; row tiles in order.
constexpr int score_blocks(int C, int kstep) {
    int n = 0;
    for (int I = 0; I < C / 16; ++I) n += (16 * (I + 1) + kstep - 1) / kstep;
    return n;
}
constexpr int score_elems(int C, int kstep) { return score_blocks(C, kstep) * 16 * kstep; }

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once
// per (kernel, device); thread-safe.  Kernels with more than 64 KiB of
// dynamic LDS need it before their first launch on each device.
hipError_t ensure_dynamic_lds(const void *kernel, int bytes);

// Launch-time profiling hooks (no-ops unless a profiling session is open).
void prof_begin(hipStream_t s);
void prof_end(hipStream_t s, const char *name);

// Kernel launchers.  They return hipSuccess or the launch error.  Shapes have
// been validated by the caller.
// coff (chunk slots) and, when ck_tokens > 0, ckoff (checkpoints of
// ck_tokens tokens each) per packed sequence
hipError_t launch_chunk_offsets(const int32_t *cu, int N, int T, int C,
                                int nc_max, int32_t *coff, int ck_tokens,
                                int32_t *ckoff, hipStream_t s);
hipError_t launch_prefill_bf16(const PrefillArgs &a, int dk, int dv, int C,
                               int bv, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs &a, int dk, int dv, int C,
                              int bv, hipStream_t s);
hipError_t launch_decode(int dtype, const void *q, const void *k,
                         const void *v, const float *g, const float *beta,
                         float *state, void *o, int N, int H, int dk, int dv,
                         hipStream_t s);
// K decode tokens per sequence from one state read: outputs only (verify;
// u_out non-null also keeps each draft's update vector, fp32 [N][K][H][dv]),
// or the first n_accept[n] tokens folded into the state (commit), or folded
// from the kept update vectors (commit_kept).
hipError_t launch_decode_verify(int dtype, const void *q, const void *k,
                                const void *v, const float *g,
                                const float *beta, const float *state,
                                void *o, float *u_out, int N, int K, int H,
                                int dk, int dv, hipStream_t s);
// The previous round's accepted drafts folded in from its kept update
// vectors (pk, pg, pu [N][Kp][H][..], pacc [N]), the committed state written,
// then K new drafts verified from it (o, and u_out when non-null).
hipError_t launch_decode_commit_verify(int dtype, const void *pk, const float *pg,
                                       const float *pu, const int32_t *pacc, int Kp,
                                       const void *q, const void *k, const void *v,
                                       const float *g, const float *beta, float *state,
                                       void *o, float *u_out, int N, int K, int H, int dk,
                                       int dv, hipStream_t s);
hipError_t launch_decode_commit_kept(int dtype, const void *k, const float *g,
                                     const float *u, const int32_t *n_accept,
                                     float *state, int N, int K, int H, int dk,
                                     int dv, hipStream_t s);
hipError_t launch_decode_commit(int dtype, const void *k, const void *v,
                                const float *g, const float *beta,
                                const int32_t *n_accept, float *state, int N,
                                int K, int H, int dk, int dv, hipStream_t s);
// Debug checks: set the device word flag_dev (null: one word shared per
// device) when g leaves [-5, 0] (bit 0) or when cu_seqlens is malformed
// (bit 1), then read it back synchronously into *flag_out.
hipError_t run_checks(const float *g, size_t n, const int32_t *cu, int N,
                      int T, unsigned *flag_dev, hipStream_t s,
                      unsigned *flag_out);

// Whether a dtype / size combination has kernels built.
bool prefill_supported(int dtype, int dk, int dv, int C);

}  // namespace kda
