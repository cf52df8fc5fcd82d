/*
 * kda.h -- C ABI of the MI355X (gfx950) Kimi Delta Attention library.
 *
 * KDA is the gated delta rule with a per-channel decay (Kimi K3 architecture
 * blog post: "Sequence" section -- three of every four layers keep a
 * fixed-size recurrent state instead of rereading the prefix; section on the
 * lower bound on the log-decay -- the state forgets as it goes, and computing
 * it chunk by chunk divides by the accumulated decay).  For one head of one
 * sequence, state S (dk x dv, fp32), per token t:
 *
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = S_t^T q_t
 *
 * Conventions for every entry point
 *   - All device pointers are caller-owned; the library never allocates device
 *     memory.  Work is enqueued on the caller's stream and the call returns
 *     without waiting, except where a flag below says otherwise.
 *   - Tensors are contiguous row-major with the shapes given below; every
 *     pointer must be 16-byte aligned (the workspace 256-byte aligned).
 *   - dk and dv are each one of 32, 64, 128.
 *   - g is the natural-log decay per channel; the method requires
 *     -5 <= g <= 0 (keep at least e^-5 = 0.67% per step, the blog post's
 *     bound, so a 16-token tile's accumulated log-decay stays in [-80, 0]).
 *     Values outside that range are undefined behaviour (they may overflow
 *     to Inf/NaN) unless KDA_FLAG_CHECK_DECAY is set.
 *   - Arguments are validated on the host before anything is enqueued; on an
 *     error nothing is launched and a negative status is returned.
 *   - q, k, v and o share one dtype (kda_dtype); g, beta and the states are
 *     always float32.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The element type of q, k, v and o.  Any int may arrive here from a C
 * caller; C++ gets the enumeration a fixed int underlying type, so every
 * such value is a valid kda_dtype there and the library's check of it
 * (KDA_ERR_UNSUPPORTED) is well defined.  Either way the type is an int. */
#ifdef __cplusplus
typedef enum kda_dtype : int {
#else
typedef enum kda_dtype {
#endif
    KDA_DTYPE_F32 = 0,  /* IEEE float32 */
    KDA_DTYPE_BF16 = 1  /* bfloat16 (outputs rounded to nearest even) */
} kda_dtype;

enum {
    KDA_OK = 0,
    KDA_ERR_NULL = -1,        /* a required pointer is NULL                     */
    KDA_ERR_SHAPE = -2,       /* a size is out of range or inconsistent         */
    KDA_ERR_UNSUPPORTED = -3, /* dk/dv/chunk/dtype combination not built        */
    KDA_ERR_WORKSPACE = -4,   /* workspace missing or smaller than required     */
    KDA_ERR_ALIGN = -5,       /* a pointer is not suitably aligned              */
    KDA_ERR_ALIAS = -6,       /* buffers overlap in a way that is not allowed   */
    KDA_ERR_LAUNCH = -7,      /* the HIP runtime reported an error              */
    KDA_ERR_DECAY_BOUND = -8, /* KDA_FLAG_CHECK_DECAY found g outside [-5, 0]   */
    KDA_ERR_TOO_LARGE = -9    /* kda_chunk_prefill_noalloc: the sizes need more
                                 scratch than its static buffer holds          */
};

/* Debug flag: before computing, scan g on the device, synchronize the stream
 * and return KDA_ERR_DECAY_BOUND (launching nothing else) if any g is
 * outside [-5, 0] or NaN.  For a packed batch it also checks that cu_seqlens
 * starts at 0, never decreases and ends at T (KDA_ERR_SHAPE otherwise).
 * This breaks the no-host-sync rule on purpose.  A checked prefill keeps its
 * result word in its own workspace; the checked decode calls (and a prefill
 * with no sequences) share one word per device, so two of those in flight
 * at once on different streams may report each other's result. */
#define KDA_FLAG_CHECK_DECAY 1u
/* Prefill: keep one state chain per (sequence, head) even when the sizes
 * would split long sequences into segments computed in parallel (the
 * blog post's serving-stack section: a sequence split across devices, each
 * part summarised by its state transition; here across compute units).
 * Results agree up to rounding either way; for comparisons and timing. */
#define KDA_FLAG_NO_SEGMENTS 2u
/* Prefill: run the whole call as one intra-chunk pass and one state pass
 * even when the sizes would split it into windows.  A fixed-length bf16
 * batch at dk = dv = 128, chunk 64 whose hand-off between the two passes
 * (72,192 bytes per (chunk, head)) comes to more than 192 MiB otherwise runs
 * as windows of at most about 160 MiB, each an intra-chunk pass followed by
 * a state pass, so that the state pass reads a hand-off the 256 MiB
 * last-level cache still holds: groups of whole sequences when one
 * sequence's hand-off fits 160 MiB, else windows over the chunks of every
 * sequence (at least 32 chunks each) with the state crossing from one to
 * the next in the workspace.  Results are bit-identical either way; for
 * comparisons and timing. */
#define KDA_FLAG_NO_WINDOWS 4u

/* Bytes of device workspace kda_chunk_prefill needs for these sizes
 * (written to *bytes).  Same arguments as kda_chunk_prefill.  The figure
 * depends only on the sizes, never on the contents of cu_seqlens. */
int kda_chunk_prefill_workspace_size(int B, int T, int H, int dk, int dv,
                                     int num_seqs, int chunk_size,
                                     kda_dtype dtype, size_t *bytes);

/*
 * Chunked KDA prefill (the blog post's chunk-wise evaluation with the decay
 * bound: every 16-token tile, the diagonal ones included, is an ordinary
 * dense matrix product).
 *
 *   q, k       [B, T, H, dk]  dtype
 *   v          [B, T, H, dv]  dtype
 *   g          [B, T, H, dk]  float32, natural-log decay in [-5, 0]
 *   beta       [B, T, H]      float32
 *   h0         [N, H, dk, dv] float32 initial state per sequence, or NULL
 *              for a zero start (prefix-cache resume: the serving-stack
 *              section restores a cached recurrent state at a boundary)
 *   cu_seqlens device int32 [N+1] or NULL.  NULL: N = B sequences of T
 *              tokens each.  Non-NULL: packed variable-length batch, B must
 *              be 1, sequence n owns rows [cu[n], cu[n+1]), cu[0] = 0 and
 *              cu[N] = T.  Malformed contents give unspecified results but
 *              never an out-of-bounds access (checked with the flag above).
 *   num_seqs   N (B when cu_seqlens is NULL)
 *   chunk_size 16 or 64 (a multiple of the 16-token tile); results are the
 *              same up to rounding.
 *   o          [B, T, H, dv]  dtype, written
 *   ht         [N, H, dk, dv] float32 final state per sequence, or NULL.
 *              ht may be exactly h0 (in-place resume); partial overlap of ht
 *              and h0, and any overlap of o/ht/workspace with an input or
 *              with each other, is KDA_ERR_ALIAS.
 *   workspace  device scratch of at least kda_chunk_prefill_workspace_size
 *              bytes, 256-byte aligned; its contents on entry do not matter.
 *              Two calls in flight on different streams need two workspaces.
 *   stream     HIP stream the kernels are enqueued on.
 * A sequence of length 0 gives ht = h0 (or zeros).  Sizes: B*T*H and N*H
 * below 2^31, and chunk_size*H*dv*4 below 2^31 (the byte span of one
 * chunk's output rows at fp32 width: H < 65536 at dv = 128, chunk 64);
 * KDA_ERR_SHAPE otherwise.
 */
int kda_chunk_prefill(const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const float *h0,
                      const int32_t *cu_seqlens, int B, int T, int H, int dk,
                      int dv, int num_seqs, int chunk_size, kda_dtype dtype,
                      unsigned flags, void *o, float *ht, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * kda_chunk_prefill for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments without a workspace.  The library keeps the
 * scratch in a static device array of KDA_NOALLOC_SCRATCH_BYTES (128 MiB)
 * that every GPU it runs on holds until the process ends; the call itself
 * allocates nothing.  Sizes whose workspace (kda_chunk_prefill_workspace_size)
 * exceeds it return KDA_ERR_TOO_LARGE before anything is enqueued; at d = 128
 * and chunk 64 that is about 1,800 (chunk, head) slots, e.g. 2048 tokens x 32
 * heads.  Every call on one GPU shares that GPU's array: calls that overlap in
 * time on one GPU (different streams or host threads) race and give
 * undefined results.  Nothing in the array needs to start at zero.  Every
 * other argument, error and result is that of kda_chunk_prefill.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (128u << 20)
int kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v,
                              const float *g, const float *beta,
                              const float *h0, const int32_t *cu_seqlens,
                              int B, int T, int H, int dk, int dv,
                              int num_seqs, int chunk_size, kda_dtype dtype,
                              unsigned flags, void *o, float *ht,
                              hipStream_t stream);

/*
 * kda_chunk_prefill that also writes strided state checkpoints, for a
 * prefix cache that restores a sequence's recurrent state at a fixed token
 * boundary (the serving-stack section of the blog post: cached states are
 * kept at block boundaries, and resuming from one is kda_chunk_prefill with
 * h0 = that checkpoint).
 *
 *   ckpt        [num_ckpt, H, dk, dv] float32, written: checkpoint j of a
 *               sequence is its state after its first (j + 1) * ckpt_stride
 *               tokens, for j = 0 .. len / ckpt_stride - 1 (integer
 *               division; a length that is an exact multiple gives a last
 *               checkpoint equal to ht).  Sequences are laid out one after
 *               another: fixed-length batches (cu_seqlens NULL) give
 *               sequence n slots n * (T / ckpt_stride) ..; packed batches
 *               give sequence n the slots after those of sequences 0..n-1.
 *               Checkpoints past num_ckpt are not written (size ckpt from
 *               the lengths: sum over sequences of len / ckpt_stride).
 *   ckpt_stride tokens between checkpoints, a positive multiple of
 *               chunk_size (else KDA_ERR_SHAPE).
 *   num_ckpt    slots in ckpt (>= 0); ckpt may be NULL only when it is 0.
 * ckpt must be 16-byte aligned and must not overlap any other argument
 * (KDA_ERR_ALIGN, KDA_ERR_ALIAS).  Every other argument, error and the
 * results o and ht are exactly those of kda_chunk_prefill; the workspace
 * size is the same.
 */
int kda_chunk_prefill_checkpointed(const void *q, const void *k,
                                   const void *v, const float *g,
                                   const float *beta, const float *h0,
                                   const int32_t *cu_seqlens, int B, int T,
                                   int H, int dk, int dv, int num_seqs,
                                   int chunk_size, kda_dtype dtype,
                                   unsigned flags, void *o, float *ht,
                                   float *ckpt, int ckpt_stride, int num_ckpt,
                                   void *workspace, size_t workspace_bytes,
                                   hipStream_t stream);

/*
 * One decode step for N independent sequences, one token each, updating the
 * state in place (the serving-stack section: the recurrent state is updated
 * in place).  Per (n, h): S' = Diag(exp(g)) S; u = beta (v - S'^T k);
 * S = S' + k u^T; o = S^T q.  The state is read once and written once.
 *
 *   q, k  [N, H, dk] dtype      v [N, H, dv] dtype
 *   g     [N, H, dk] float32    beta [N, H] float32
 *   state [N, H, dk, dv] float32, read and overwritten
 *   o     [N, H, dv] dtype, written; must not overlap any other argument
 */
int kda_decode_step(const void *q, const void *k, const void *v,
                    const float *g, const float *beta, float *state, void *o,
                    int N, int H, int dk, int dv, kda_dtype dtype,
                    unsigned flags, hipStream_t stream);

/*
 * Speculative decoding (the serving-stack section of the blog post: K
 * drafted tokens are checked in one pass from the committed recurrent
 * state, rebuilt on chip from the cached per-token inputs, then the
 * accepted prefix is committed).  Every call reads each (sequence, head)
 * state from HBM once; verify, verify_keep and commit apply the decode
 * step's arithmetic token by token with the state held on chip,
 * commit_kept applies the accepted drafts in closed form from the update
 * vectors verify_keep kept, and commit_verify folds one round's commit into
 * the next round's verify.  Token t of sequence n is row n * K + t of the
 * [N, K, H, d] inputs.
 *
 * kda_decode_verify: outputs of all K tokens; the state is only read.
 *   q, k  [N, K, H, dk] dtype   v [N, K, H, dv] dtype
 *   g     [N, K, H, dk] float32 beta [N, K, H] float32
 *   state [N, H, dk, dv] float32, read only (the committed state)
 *   o     [N, K, H, dv] dtype, written; must not overlap any input
 *         o[n, t] equals what t + 1 consecutive kda_decode_step calls on a
 *         copy of the state would give for token t.
 */
int kda_decode_verify(const void *q, const void *k, const void *v,
                      const float *g, const float *beta, const float *state,
                      void *o, int N, int K, int H, int dk, int dv,
                      kda_dtype dtype, unsigned flags, hipStream_t stream);

/*
 * kda_decode_commit: folds the first n_accept[n] draft tokens of each
 * sequence into its state, in place (values are clamped to [0, K]; 0
 * leaves the state untouched).  k, v, g, beta as in kda_decode_verify (q is
 * not needed); n_accept device int32 [N]; state [N, H, dk, dv] float32, read
 * and written; it must not overlap any input.
 */
int kda_decode_commit(const void *k, const void *v, const float *g,
                      const float *beta, const int32_t *n_accept,
                      float *state, int N, int K, int H, int dk, int dv,
                      kda_dtype dtype, unsigned flags, hipStream_t stream);

/*
 * kda_decode_verify_keep: kda_decode_verify that also keeps, for every draft
 * token, its update vector u_t = beta_t (v_t - S'^T k_t) (the value the
 * recurrence adds along k_t, S' the state decayed by e^{g_t} after drafts
 * 0..t-1), so that a commit need not recompute it.
 *   inputs and o as in kda_decode_verify
 *   u     [N, K, H, dv] float32, written; must not overlap any input or o
 * o is bit-identical to kda_decode_verify's.
 */
int kda_decode_verify_keep(const void *q, const void *k, const void *v,
                           const float *g, const float *beta,
                           const float *state, void *o, float *u, int N,
                           int K, int H, int dk, int dv, kda_dtype dtype,
                           unsigned flags, hipStream_t stream);

/*
 * kda_decode_commit_kept: kda_decode_commit from the update vectors that
 * kda_decode_verify_keep kept on the same committed state and drafts: with
 * D_t the per-row product of e^g over drafts t .. n-1, the state after the
 * first n drafts is Diag(D_0) S + sum_{t<n} Diag(D_{t+1}) k_t u_t^T, one
 * streaming pass over the state with no reduction over dk (same result as
 * kda_decode_commit up to rounding order).  If the state changed since the
 * verify, the result is not that of the drafts.
 *   k [N, K, H, dk] dtype; g [N, K, H, dk] float32; u [N, K, H, dv] float32
 *   n_accept device int32 [N], clamped to [0, K] (0 leaves the state as is)
 *   state [N, H, dk, dv] float32, read and written in place; it must not
 *   overlap any input.
 */
int kda_decode_commit_kept(const void *k, const float *g, const float *u,
                           const int32_t *n_accept, float *state, int N, int K,
                           int H, int dk, int dv, kda_dtype dtype,
                           unsigned flags, hipStream_t stream);

/*
 * kda_decode_commit_verify: one round of a speculative loop in one pass over
 * the states: the previous round's accepted drafts are committed from the
 * update vectors its verify kept (as kda_decode_commit_kept would, token by
 * token with u known), the committed state is written, and K new drafts are
 * verified from it (as kda_decode_verify_keep would).  Each state is read
 * once and, when its sequence accepted a draft, written once.
 *   prev_k [N, Kp, H, dk] dtype; prev_g [N, Kp, H, dk] float32;
 *   prev_u [N, Kp, H, dv] float32 (kept by the previous round's verify on
 *   this same state); n_accept device int32 [N], clamped to [0, Kp]; all
 *   may be null when Kp == 0 (nothing to commit)
 *   q, k, v, g, beta, o as in kda_decode_verify (may be null when K == 0:
 *   commit only)
 *   u     [N, K, H, dv] float32 or null: the new drafts' update vectors, for
 *         the next round
 *   state [N, H, dk, dv] float32, read and written in place; state, o and u
 *         must not overlap each other or any input.
 * The committed state equals kda_decode_commit's bit for bit when the
 * previous round's u was kept from the same state, and o (and u) then equal
 * kda_decode_verify_keep's from that committed state.
 */
int kda_decode_commit_verify(const void *prev_k, const float *prev_g,
                             const float *prev_u, const int32_t *n_accept,
                             int Kp, const void *q, const void *k,
                             const void *v, const float *g, const float *beta,
                             float *state, void *o, float *u, int N, int K,
                             int H, int dk, int dv, kda_dtype dtype,
                             unsigned flags, hipStream_t stream);

/* Static, human-readable text for a status code. */
const char *kda_status_string(int status);

/* ---------------------------------------------------------------------
 * Launch timing (measurement plumbing).  Between kda_profile_start and
 * kda_profile_stop every kernel the library enqueues is bracketed by a pair
 * of HIP events recorded on the same stream (no host synchronisation).
 * kda_profile_stop synchronizes on the recorded events and reports, per
 * kernel name, the number of launches and their summed duration.  Launches
 * beyond max_launches are not timed.  Not thread-safe; one session at a
 * time per process.
 * --------------------------------------------------------------------- */
typedef struct kda_kernel_time {
    char name[48];
    int launches;
    double total_ms;
} kda_kernel_time;

int kda_profile_start(int max_launches);
int kda_profile_stop(kda_kernel_time *out, int max_entries, int *n_entries);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
