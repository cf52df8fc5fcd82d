// C ABI of the KDA library: host-side validation, workspace carve-up,
// dispatch to the gfx950 kernels, and launch timing.  No device memory is
// ever allocated here; every buffer belongs to the caller.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <utility>
#include <string>
#include <vector>

#include "../../include/kda.h"
#include "kda_launch.h"

namespace kda {

static size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

SegPlan seg_plan(bool packed, int dtype, int dk, int dv, int C, int N, int H, int nc_seq) {
    // worth it when the chains (32-column blocks) number under half a device
    // of compute units and the sequences are long; each segment keeps at
    // least 8 chunks, and the segments aim at ~1024 chains in all.  "Long"
    // depends on the single chain it replaces: the loader-fed chain (bf16,
    // dk = dv = 128, chunk 64) keeps up until at least 128 chunks and three
    // chunks per 32-column chain (measured: 64 chunks 0.84-0.93x, H = 16 at
    // 128 chunks 0.84x, 128 chunks at up to 32 chains 1.05-1.15x), the other
    // chains until 64 chunks
    const int64_t chains = int64_t(N) * H * (dv >= 32 ? dv / 32 : 1);
    const bool loader_fed = dtype == KDA_DTYPE_BF16 && dk == 128 && dv == 128 && C == 64;
    const int64_t min_nc = loader_fed ? std::max<int64_t>(128, 3 * chains) : 64;
    if (packed || chains <= 0 || chains >= 128 || nc_seq < min_nc) return SegPlan{1, 0};
    int64_t nseg = (1024 + chains - 1) / chains;
    if (nseg > nc_seq / 8) nseg = nc_seq / 8;
    if (nseg < 2) return SegPlan{1, 0};
    const int seg_len = int((nc_seq + nseg - 1) / nseg);
    return SegPlan{(nc_seq + seg_len - 1) / seg_len, seg_len};
}

size_t handoff_slot_bytes(int dk, int dv, int C, size_t elem_bytes) {
    return (size_t(C) * dk * 2 + size_t(chunk_pad(C, elem_bytes)) * dk + size_t(C) * dv +
            size_t(score_elems(C, elem_bytes == 2 ? 32 : 4))) * elem_bytes + size_t(dk) * sizeof(float);
}

WinPlan win_plan(bool packed, int dtype, int dk, int dv, int C, int N, int H, int nc_seq, int nseg) {
    // The state pass reads the hand-off the intra-chunk pass wrote; it runs
    // 15-18% faster when that hand-off is still in the 256 MiB last-level
    // cache.  Once the hand-off passes 192 MiB the call runs as windows of
    // about 160 MiB: groups of whole sequences, or, for a sequence larger
    // than that, windows over its chunks (with the state carried between
    // them), provided each keeps at least 32 of its chunks: a state chain of
    // fewer does not repay its pipeline fill (measured: 16 chunks even, 8
    // slower).  Each window costs a launch pair.
    const WinPlan none{N, 1};
    const bool loader_fed = dtype == KDA_DTYPE_BF16 && dk == 128 && dv == 128 && C == 64;
    if (packed || !loader_fed || nseg > 1 || nc_seq < 1 || N < 1) return none;
    const double mib_seq = double(nc_seq) * H * double(handoff_slot_bytes(dk, dv, C, 2)) / double(1 << 20);
    if (mib_seq * N <= 192.0) return none;
    if (mib_seq <= 160.0) {
        const int grp = int(160.0 / mib_seq);
        return grp >= N ? none : WinPlan{grp, 1};
    }
    const int nchunk = int(mib_seq / 160.0 + 0.999);
    return nc_seq / nchunk >= 32 ? WinPlan{1, nchunk} : none;
}

PrefillLayout prefill_layout(int nc_max, int H, int N, int dk, int dv, int C, size_t elem_bytes, int nseg,
                             bool carry) {
    PrefillLayout L;
    const size_t slots = size_t(nc_max) * size_t(H);
    size_t off = 0;
    L.coff = off;
    off = align_up(off + sizeof(int32_t) * size_t(N + 1), 256);
    L.ckoff = off;
    off = align_up(off + sizeof(int32_t) * size_t(N + 1), 256);
    L.W = off;
    off = align_up(off + slots * C * dk * elem_bytes, 256);
    L.Qg = off;
    off = align_up(off + slots * C * dk * elem_bytes, 256);
    L.KtT = off;
    off = align_up(off + slots * chunk_pad(C, elem_bytes) * dk * elem_bytes, 256);
    L.Ut = off;
    off = align_up(off + slots * C * dv * elem_bytes, 256);
    L.Ps = off;
    off = align_up(off + slots * score_elems(C, elem_bytes == 2 ? 32 : 4) * elem_bytes, 256);
    L.D = off;
    off = align_up(off + slots * dk * sizeof(float), 256);
    const size_t sch = nseg > 1 ? size_t(N) * nseg * H : 0;  // segment chains
    L.Mseg = off;
    off = align_up(off + sch * dk * dk * sizeof(float), 256);
    L.Bseg = off;
    off = align_up(off + sch * dk * dv * sizeof(float), 256);
    L.Sin = off;
    off = align_up(off + sch * dk * dv * sizeof(float), 256);
    L.carry = off;  // the state between chunk windows
    off = align_up(off + (carry ? size_t(N) * H * dk * dv * sizeof(float) : 0), 256);
    L.dummy = off;
    off += 1024;
    L.flag = off;  // result word of the checked mode
    off += 256;
    L.total = off;
    return L;
}

bool prefill_supported(int dtype, int dk, int dv, int C) {
    auto okd = [](int d) { return d == 32 || d == 64 || d == 128; };
    if (!okd(dk) || !okd(dv) || (C != 16 && C != 64)) return false;
    return dtype == KDA_DTYPE_F32 || dtype == KDA_DTYPE_BF16;
}

// ------------------------------------------------------------------ timing
namespace {
struct ProfRec {
    hipEvent_t start, stop;
    std::string name;
};
struct Profiler {
    bool active = false;
    int cap = 0;
    int used = 0;
    std::vector<hipEvent_t> evs;  // 2 * cap events, created up front
    std::vector<std::string> names;
} g_prof;
}  // namespace

hipError_t ensure_dynamic_lds(const void *kernel, int bytes) {
    static std::mutex mu;
    static std::vector<std::pair<const void *, int>> done;  // (kernel, device)
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    for (const auto &d : done)
        if (d.first == kernel && d.second == dev) return hipSuccess;
    e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done.emplace_back(kernel, dev);
    return e;
}

void prof_begin(hipStream_t s) {
    if (!g_prof.active || g_prof.used >= g_prof.cap) return;
    (void)hipEventRecord(g_prof.evs[2 * g_prof.used], s);
}

void prof_end(hipStream_t s, const char *name) {
    if (!g_prof.active || g_prof.used >= g_prof.cap) return;
    (void)hipEventRecord(g_prof.evs[2 * g_prof.used + 1], s);
    g_prof.names[g_prof.used] = name;
    ++g_prof.used;
}

}  // namespace kda

using namespace kda;

// Compute units of the current device, queried once per device.
static int device_cu_count() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
    if (dev < 64 && cached[dev] > 0) return cached[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev < 64) cached[dev] = n;
    return n;
}

static bool misaligned(const void *p, size_t a) { return p && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

static bool overlap(const void *a, size_t na, const void *b, size_t nb) {
    if (!a || !b || na == 0 || nb == 0) return false;
    const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
    return x < y + nb && y < x + na;
}

static size_t dtype_bytes(kda_dtype dt) { return dt == KDA_DTYPE_BF16 ? 2 : 4; }

// ---------------------------------------------------------------------------
// Scratch of kda_chunk_prefill_noalloc: a static device array, one copy per
// GPU, held until the process ends.  In host code its name is only a
// host-side stand-in: the device address of each GPU's copy is looked up
// once per device (with that device current) and used everywhere instead.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[KDA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];
}  // namespace

// This device's copy of the scratch array (status KDA_OK), looked up on the
// first call made with the device current.
static int device_scratch(void **out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KDA_ERR_LAUNCH;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return KDA_ERR_LAUNCH;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return KDA_OK;
}

extern "C" {

const char *kda_status_string(int status) {
    switch (status) {
    case KDA_OK: return "ok";
    case KDA_ERR_NULL: return "a required pointer is NULL";
    case KDA_ERR_SHAPE: return "a size is out of range or inconsistent";
    case KDA_ERR_UNSUPPORTED: return "unsupported dk/dv/chunk/dtype combination";
    case KDA_ERR_WORKSPACE: return "workspace missing or too small";
    case KDA_ERR_ALIGN: return "a pointer is not suitably aligned";
    case KDA_ERR_ALIAS: return "buffers overlap in a way that is not allowed";
    case KDA_ERR_LAUNCH: return "the HIP runtime reported an error";
    case KDA_ERR_DECAY_BOUND: return "a log-decay value is outside [-5, 0]";
    case KDA_ERR_TOO_LARGE: return "the sizes need more scratch than the static buffer holds";
    default: return "unknown status";
    }
}

// Shared shape checks; fills nc_max and N (number of sequences).
static int prefill_shape(int B, int T, int H, int dk, int dv, int num_seqs, int chunk_size, kda_dtype dt,
                         bool packed, int *nc_max, int *N) {
    if (dt != KDA_DTYPE_F32 && dt != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
    if (B < 0 || T < 0 || H <= 0 || num_seqs < 0) return KDA_ERR_SHAPE;
    if (!prefill_supported(dt, dk, dv, chunk_size)) return KDA_ERR_UNSUPPORTED;
    if (packed) {
        if (B != 1) return KDA_ERR_SHAPE;
        *N = num_seqs;
        const int64_t slots = (int64_t(T) + chunk_size - 1) / chunk_size + num_seqs;
        if (slots > INT32_MAX / 2) return KDA_ERR_SHAPE;
        *nc_max = int(slots);
    } else {
        if (num_seqs != B) return KDA_ERR_SHAPE;
        *N = B;
        const int64_t slots = int64_t(B) * ((int64_t(T) + chunk_size - 1) / chunk_size);
        if (slots > INT32_MAX / 2) return KDA_ERR_SHAPE;
        *nc_max = int(slots);
    }
    // element offsets are computed in 64 bits; per-dimension products in 32,
    // and so are the byte offsets of one chunk's output rows (up to C rows of
    // H x dv values), which the range-checked o stores take as 32-bit offsets
    if (int64_t(B) * T * H > INT32_MAX || int64_t(*N) * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (int64_t(chunk_size) * H * dv * 4 > INT32_MAX) return KDA_ERR_SHAPE;
    return KDA_OK;
}

int kda_chunk_prefill_workspace_size(int B, int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                                     kda_dtype dtype, size_t *bytes) {
    if (!bytes) return KDA_ERR_NULL;
    // the size must not depend on whether cu_seqlens is given: take the
    // larger of the two slot counts
    int nc_a = 0, nc_b = 0, N = 0, st;
    if (B == 1) {
        st = prefill_shape(B, T, H, dk, dv, num_seqs, chunk_size, dtype, true, &nc_a, &N);
        if (st != KDA_OK) return st;
    }
    if (num_seqs == B) {
        st = prefill_shape(B, T, H, dk, dv, num_seqs, chunk_size, dtype, false, &nc_b, &N);
        if (st != KDA_OK) return st;
    } else if (B != 1) {
        return KDA_ERR_SHAPE;
    }
    const int nc = std::max(nc_a, nc_b);
    // segment buffers when the fixed-length reading of these sizes segments,
    // the window carry when it runs in windows
    const int ncs = (T + chunk_size - 1) / chunk_size;
    const int nseg = (num_seqs == B) ? seg_plan(false, dtype, dk, dv, chunk_size, B, H, ncs).nseg : 1;
    const bool carry = num_seqs == B && win_plan(false, dtype, dk, dv, chunk_size, B, H, ncs, nseg).nchunk > 1;
    *bytes = prefill_layout(nc, H, num_seqs, dk, dv, chunk_size, dtype_bytes(dtype), nseg, carry).total;
    return KDA_OK;
}

namespace {

// Optional strided checkpoints of a prefill call (ckpt null: none).
struct CkptReq {
    float *ckpt;
    int stride, num_ckpt;
};

int prefill_impl(const void *q, const void *k, const void *v, const float *g, const float *beta, const float *h0,
                 const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv, int num_seqs, int chunk_size,
                 kda_dtype dtype, unsigned flags, void *o, float *ht, void *workspace, size_t workspace_bytes,
                 hipStream_t stream, const CkptReq &ck) {
    const bool packed = cu_seqlens != nullptr;
    int nc_max = 0, N = 0;
    int st = prefill_shape(B, T, H, dk, dv, num_seqs, chunk_size, dtype, packed, &nc_max, &N);
    if (st != KDA_OK) return st;
    const size_t rows = size_t(B) * size_t(T);
    const size_t eb = dtype_bytes(dtype);
    const bool any_tokens = rows > 0;
    if (any_tokens && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    if (!workspace && N > 0) return KDA_ERR_WORKSPACE;

    size_t need = 0;
    st = kda_chunk_prefill_workspace_size(B, T, H, dk, dv, num_seqs, chunk_size, dtype, &need);
    if (st != KDA_OK) return st;
    if (N > 0 && workspace_bytes < need) return KDA_ERR_WORKSPACE;

    for (const void *p : {q, k, v, (const void *)g, (const void *)beta, (const void *)h0, (const void *)o,
                          (const void *)ht, (const void *)cu_seqlens, (const void *)ck.ckpt})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    if (misaligned(workspace, 256)) return KDA_ERR_ALIGN;

    const size_t nq = rows * H * dk * eb, nv = rows * H * dv * eb, ng = rows * H * dk * 4, nb = rows * H * 4;
    const size_t ns = size_t(N) * H * dk * dv * 4;
    const size_t ncu = packed ? sizeof(int32_t) * size_t(N + 1) : 0;
    const size_t nck = size_t(ck.num_ckpt) * H * dk * dv * 4;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{q, nq}, {k, nq}, {v, nv}, {g, ng}, {beta, nb}, {h0, ns}, {cu_seqlens, ncu}};
    const Buf outs[] = {{o, nv}, {ht, ns}, {workspace, need}, {ck.ckpt, nck}};
    constexpr int NOUT = 4;
    for (int i = 0; i < NOUT; ++i) {
        for (const Buf &b : ins) {
            if (i == 1 && b.p == h0) {  // ht == h0 exactly is an in-place resume
                if (ht && h0 && ht != h0 && overlap(ht, ns, h0, ns)) return KDA_ERR_ALIAS;
                continue;
            }
            if (overlap(outs[i].p, outs[i].n, b.p, b.n)) return KDA_ERR_ALIAS;
        }
        for (int j = i + 1; j < NOUT; ++j)
            if (overlap(outs[i].p, outs[i].n, outs[j].p, outs[j].n)) return KDA_ERR_ALIAS;
    }

    if (N == 0) {
        // nothing to compute (the workspace may be absent); the checked mode
        // still screens the inputs, with the device's shared result word
        if (flags & KDA_FLAG_CHECK_DECAY) {
            unsigned flag = 0;
            if (run_checks(g, rows * H * dk, cu_seqlens, N, T, nullptr, stream, &flag) != hipSuccess)
                return KDA_ERR_LAUNCH;
            if (flag & 2u) return KDA_ERR_SHAPE;
            if (flag & 1u) return KDA_ERR_DECAY_BOUND;
        }
        return KDA_OK;
    }

    const SegPlan sp = (flags & KDA_FLAG_NO_SEGMENTS) ? SegPlan{1, 0}
                                                     : seg_plan(packed, dtype, dk, dv, chunk_size, N, H,
                                                                (T + chunk_size - 1) / chunk_size);
    // the layout is the one the size query computed (segment buffers present
    // whenever the sizes call for them, also when a flag turns them off)
    const SegPlan sp_ws = seg_plan(packed, dtype, dk, dv, chunk_size, N, H, (T + chunk_size - 1) / chunk_size);
    const WinPlan wp = win_plan(packed, dtype, dk, dv, chunk_size, N, H, (T + chunk_size - 1) / chunk_size, sp_ws.nseg);
    const PrefillLayout L = prefill_layout(nc_max, H, N, dk, dv, chunk_size, eb, sp_ws.nseg, wp.nchunk > 1);
    unsigned char *ws = static_cast<unsigned char *>(workspace);
    if (flags & KDA_FLAG_CHECK_DECAY) {
        // the result word is this call's own (in its workspace)
        unsigned flag = 0;
        if (run_checks(g, rows * H * dk, cu_seqlens, N, T, reinterpret_cast<unsigned *>(ws + L.flag), stream,
                       &flag) != hipSuccess)
            return KDA_ERR_LAUNCH;
        if (flag & 2u) return KDA_ERR_SHAPE;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    PrefillArgs a;
    a.q = q; a.k = k; a.v = v; a.g = g; a.beta = beta; a.h0 = h0;
    a.cu = cu_seqlens;
    a.coff = reinterpret_cast<int32_t *>(ws + L.coff);
    a.T = T; a.H = H; a.N = N;
    a.nc_max = nc_max;
    a.nc_seq = (T + chunk_size - 1) / chunk_size;
    a.num_cu = device_cu_count();
    if (a.num_cu <= 0) return KDA_ERR_LAUNCH;
    a.o = o; a.ht = ht;
    a.W = ws + L.W; a.Qg = ws + L.Qg; a.KtT = ws + L.KtT; a.Ut = ws + L.Ut; a.Ps = ws + L.Ps;
    a.D = reinterpret_cast<float *>(ws + L.D);
    a.dummy = ws + L.dummy;
    const bool want_ck = ck.ckpt && ck.num_ckpt > 0;
    a.ckpt = want_ck ? ck.ckpt : nullptr;
    a.ckoff = reinterpret_cast<int32_t *>(ws + L.ckoff);
    a.ck_every = want_ck ? ck.stride / chunk_size : 1;
    a.ck_per_seq = (want_ck && !packed) ? T / ck.stride : 0;
    a.num_ckpt = want_ck ? ck.num_ckpt : 0;
    a.seg_len = sp.seg_len;
    a.nseg = sp.nseg;
    a.Mseg = reinterpret_cast<float *>(ws + L.Mseg);
    a.Bseg = reinterpret_cast<float *>(ws + L.Bseg);
    a.Sin = reinterpret_cast<float *>(ws + L.Sin);
    // windows: the size plan's, unless a flag turned them or the segments off
    // (the carry is in the workspace whenever the plan has chunk windows)
    const bool win = (wp.grp < N || wp.nchunk > 1) && sp.nseg == 1 && !(flags & KDA_FLAG_NO_WINDOWS);
    a.win_grp = win ? wp.grp : N;
    a.win_len = win ? (a.nc_seq + wp.nchunk - 1) / wp.nchunk : a.nc_seq;
    a.nwin = win ? ((N + a.win_grp - 1) / a.win_grp) * ((a.nc_seq + a.win_len - 1) / a.win_len) : 1;
    a.win_n0 = 0;
    a.win_nn = N;
    a.win_c0 = 0;
    a.win_nc = a.nc_seq;
    a.carry = reinterpret_cast<float *>(ws + L.carry);

    if (!any_tokens) a.nc_max = 0;  // only the state copy h0 -> ht remains
    if (packed && a.nc_max > 0) {
        if (launch_chunk_offsets(cu_seqlens, N, T, chunk_size, nc_max, a.coff, want_ck ? ck.stride : 0, a.ckoff,
                                 stream) != hipSuccess)
            return KDA_ERR_LAUNCH;
    }
    if (packed && a.nc_max == 0) {
        // no tokens at all: every sequence is empty; the state kernel still
        // runs (with zero chunks) to write ht = h0
        a.cu = nullptr;
        a.nc_seq = 0;
        a.win_nc = 0;
        a.win_len = 0;
        a.nwin = 1;
        a.win_grp = N;
        a.T = 0;
        a.ckpt = nullptr;
        a.ck_per_seq = 0;
        a.seg_len = 0;
        a.nseg = 1;
    }
    if (!any_tokens) {
        a.seg_len = 0;
        a.nseg = 1;
        a.nwin = 1;
    }
    // value-column block: narrow blocks when few (sequence, head) chains
    // would leave compute units idle; bf16 at dk = dv = 128, chunk 64 always
    // takes 16 columns, the loader-fed chain (measured faster than 32-column
    // register-fed blocks at many chains too: 1411 vs 1445 us over 64
    // sequences of 256 to 4096 tokens, 16 heads)
    const bool loader_fed = dtype == KDA_DTYPE_BF16 && dk == 128 && dv == 128 && chunk_size == 64;
    const int bv = (loader_fed || int64_t(N) * H * (dv / 32) < 512) ? 16 : 32;
    a.fd_H = make_fastdiv(uint32_t(a.H));
    a.fd_nc_seq = make_fastdiv(uint32_t(a.nc_seq));
    a.fd_win_nn = make_fastdiv(uint32_t(a.win_nn));
    hipError_t e = (dtype == KDA_DTYPE_BF16) ? launch_prefill_bf16(a, dk, dv, chunk_size, bv, stream)
                                             : launch_prefill_f32(a, dk, dv, chunk_size, bv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

}  // namespace

int kda_chunk_prefill(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const float *h0, const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                      int num_seqs, int chunk_size, kda_dtype dtype, unsigned flags, void *o, float *ht,
                      void *workspace, size_t workspace_bytes, hipStream_t stream) {
    return prefill_impl(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size, dtype, flags, o,
                        ht, workspace, workspace_bytes, stream, CkptReq{nullptr, 0, 0});
}

int kda_chunk_prefill_checkpointed(const void *q, const void *k, const void *v, const float *g,
                                   const float *beta, const float *h0, const int32_t *cu_seqlens, int B, int T,
                                   int H, int dk, int dv, int num_seqs, int chunk_size, kda_dtype dtype,
                                   unsigned flags, void *o, float *ht, float *ckpt, int ckpt_stride,
                                   int num_ckpt, void *workspace, size_t workspace_bytes, hipStream_t stream) {
    if (num_ckpt < 0 || ckpt_stride <= 0 || chunk_size <= 0 || ckpt_stride % chunk_size != 0) return KDA_ERR_SHAPE;
    if (num_ckpt > 0 && !ckpt) return KDA_ERR_NULL;
    return prefill_impl(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size, dtype, flags, o,
                        ht, workspace, workspace_bytes, stream, CkptReq{ckpt, ckpt_stride, num_ckpt});
}

int kda_chunk_prefill_noalloc(const void *q, const void *k, const void *v, const float *g, const float *beta,
                              const float *h0, const int32_t *cu_seqlens, int B, int T, int H, int dk, int dv,
                              int num_seqs, int chunk_size, kda_dtype dtype, unsigned flags, void *o, float *ht,
                              hipStream_t stream) {
    // the shape errors of kda_chunk_prefill first, then the scratch limit,
    // both before the device is touched
    int nc_max = 0, N = 0;
    int st = prefill_shape(B, T, H, dk, dv, num_seqs, chunk_size, dtype, cu_seqlens != nullptr, &nc_max, &N);
    if (st != KDA_OK) return st;
    size_t need = 0;
    st = kda_chunk_prefill_workspace_size(B, T, H, dk, dv, num_seqs, chunk_size, dtype, &need);
    if (st != KDA_OK) return st;
    if (need > size_t(KDA_NOALLOC_SCRATCH_BYTES)) return KDA_ERR_TOO_LARGE;
    void *ws = nullptr;
    st = device_scratch(&ws);
    if (st != KDA_OK) return st;
    // nothing in the scratch needs to start at zero: every word a kernel
    // reads there is written earlier in the same call
    return prefill_impl(q, k, v, g, beta, h0, cu_seqlens, B, T, H, dk, dv, num_seqs, chunk_size, dtype, flags, o,
                        ht, ws, size_t(KDA_NOALLOC_SCRATCH_BYTES), stream, CkptReq{nullptr, 0, 0});
}

int kda_decode_step(const void *q, const void *k, const void *v, const float *g, const float *beta,
                    float *state, void *o, int N, int H, int dk, int dv, kda_dtype dtype, unsigned flags,
                    hipStream_t stream) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || H <= 0) return KDA_ERR_SHAPE;
    auto okd = [](int d) { return d == 32 || d == 64 || d == 128; };
    if (!okd(dk) || !okd(dv)) return KDA_ERR_UNSUPPORTED;
    if (int64_t(N) * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)g, (const void *)beta, (const void *)state, (const void *)o})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    const size_t nh = size_t(N) * H, eb = dtype_bytes(dtype);
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{q, nh * dk * eb}, {k, nh * dk * eb}, {v, nh * dv * eb}, {g, nh * dk * 4}, {beta, nh * 4}};
    const size_t nstate = nh * dk * dv * 4, no = nh * dv * eb;
    for (const Buf &b : ins) {
        if (overlap(state, nstate, b.p, b.n) || overlap(o, no, b.p, b.n)) return KDA_ERR_ALIAS;
    }
    if (overlap(state, nstate, o, no)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {
        unsigned flag = 0;
        if (run_checks(g, nh * dk, nullptr, 0, 0, nullptr, stream, &flag) != hipSuccess) return KDA_ERR_LAUNCH;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    hipError_t e = launch_decode(dtype == KDA_DTYPE_BF16 ? 1 : 0, q, k, v, g, beta, state, o, N, H, dk, dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

namespace {

// Shared checks of the multi-token decode calls.
int decode_multi_shape(int N, int K, int H, int dk, int dv, kda_dtype dtype) {
    if (dtype != KDA_DTYPE_F32 && dtype != KDA_DTYPE_BF16) return KDA_ERR_UNSUPPORTED;
    if (N < 0 || K < 0 || H <= 0) return KDA_ERR_SHAPE;
    auto okd = [](int d) { return d == 32 || d == 64 || d == 128; };
    if (!okd(dk) || !okd(dv)) return KDA_ERR_UNSUPPORTED;
    if (int64_t(N) * H > INT32_MAX || int64_t(N) * K * H > INT32_MAX) return KDA_ERR_SHAPE;
    return KDA_OK;
}

}  // namespace

int kda_decode_verify(const void *q, const void *k, const void *v, const float *g, const float *beta,
                      const float *state, void *o, int N, int K, int H, int dk, int dv, kda_dtype dtype,
                      unsigned flags, hipStream_t stream) {
    int st = decode_multi_shape(N, K, H, dk, dv, dtype);
    if (st != KDA_OK) return st;
    if (N == 0 || K == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o) return KDA_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)g, (const void *)beta, (const void *)state, (const void *)o})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    const size_t rows = size_t(N) * K * H, eb = dtype_bytes(dtype);
    const size_t nstate = size_t(N) * H * dk * dv * 4, no = rows * dv * eb;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{q, rows * dk * eb}, {k, rows * dk * eb}, {v, rows * dv * eb}, {g, rows * dk * 4},
                       {beta, rows * 4}, {state, nstate}};
    for (const Buf &b : ins)
        if (overlap(o, no, b.p, b.n)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {
        unsigned flag = 0;
        if (run_checks(g, rows * dk, nullptr, 0, 0, nullptr, stream, &flag) != hipSuccess) return KDA_ERR_LAUNCH;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    hipError_t e = launch_decode_verify(dtype == KDA_DTYPE_BF16 ? 1 : 0, q, k, v, g, beta, state, o, nullptr, N, K,
                                        H, dk, dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_decode_verify_keep(const void *q, const void *k, const void *v, const float *g, const float *beta,
                           const float *state, void *o, float *u, int N, int K, int H, int dk, int dv,
                           kda_dtype dtype, unsigned flags, hipStream_t stream) {
    int st = decode_multi_shape(N, K, H, dk, dv, dtype);
    if (st != KDA_OK) return st;
    if (N == 0 || K == 0) return KDA_OK;
    if (!q || !k || !v || !g || !beta || !state || !o || !u) return KDA_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)g, (const void *)beta, (const void *)state, (const void *)o,
                          (const void *)u})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    const size_t rows = size_t(N) * K * H, eb = dtype_bytes(dtype);
    const size_t nstate = size_t(N) * H * dk * dv * 4, no = rows * dv * eb, nu = rows * dv * 4;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{q, rows * dk * eb}, {k, rows * dk * eb}, {v, rows * dv * eb}, {g, rows * dk * 4},
                       {beta, rows * 4}, {state, nstate}};
    for (const Buf &b : ins)
        if (overlap(o, no, b.p, b.n) || overlap(u, nu, b.p, b.n)) return KDA_ERR_ALIAS;
    if (overlap(o, no, u, nu)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {
        unsigned flag = 0;
        if (run_checks(g, rows * dk, nullptr, 0, 0, nullptr, stream, &flag) != hipSuccess) return KDA_ERR_LAUNCH;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    hipError_t e = launch_decode_verify(dtype == KDA_DTYPE_BF16 ? 1 : 0, q, k, v, g, beta, state, o, u, N, K, H, dk,
                                        dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_decode_commit(const void *k, const void *v, const float *g, const float *beta, const int32_t *n_accept,
                      float *state, int N, int K, int H, int dk, int dv, kda_dtype dtype, unsigned flags,
                      hipStream_t stream) {
    int st = decode_multi_shape(N, K, H, dk, dv, dtype);
    if (st != KDA_OK) return st;
    if (N == 0 || K == 0) return KDA_OK;
    if (!k || !v || !g || !beta || !n_accept || !state) return KDA_ERR_NULL;
    for (const void *p : {k, v, (const void *)g, (const void *)beta, (const void *)state})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    if (misaligned(n_accept, 4)) return KDA_ERR_ALIGN;
    const size_t rows = size_t(N) * K * H, eb = dtype_bytes(dtype);
    const size_t nstate = size_t(N) * H * dk * dv * 4;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{k, rows * dk * eb}, {v, rows * dv * eb}, {g, rows * dk * 4}, {beta, rows * 4},
                       {n_accept, size_t(N) * 4}};
    for (const Buf &b : ins)
        if (overlap(state, nstate, b.p, b.n)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {
        unsigned flag = 0;
        if (run_checks(g, rows * dk, nullptr, 0, 0, nullptr, stream, &flag) != hipSuccess) return KDA_ERR_LAUNCH;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    hipError_t e = launch_decode_commit(dtype == KDA_DTYPE_BF16 ? 1 : 0, k, v, g, beta, n_accept, state, N, K, H,
                                        dk, dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_decode_commit_kept(const void *k, const float *g, const float *u, const int32_t *n_accept, float *state,
                           int N, int K, int H, int dk, int dv, kda_dtype dtype, unsigned flags, hipStream_t stream) {
    int st = decode_multi_shape(N, K, H, dk, dv, dtype);
    if (st != KDA_OK) return st;
    if (N == 0 || K == 0) return KDA_OK;
    if (!k || !g || !u || !n_accept || !state) return KDA_ERR_NULL;
    for (const void *p : {k, (const void *)g, (const void *)u, (const void *)state})
        if (misaligned(p, 16)) return KDA_ERR_ALIGN;
    if (misaligned(n_accept, 4)) return KDA_ERR_ALIGN;
    const size_t rows = size_t(N) * K * H, eb = dtype_bytes(dtype);
    const size_t nstate = size_t(N) * H * dk * dv * 4;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{k, rows * dk * eb}, {g, rows * dk * 4}, {u, rows * dv * 4}, {n_accept, size_t(N) * 4}};
    for (const Buf &b : ins)
        if (overlap(state, nstate, b.p, b.n)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {
        unsigned flag = 0;
        if (run_checks(g, rows * dk, nullptr, 0, 0, nullptr, stream, &flag) != hipSuccess) return KDA_ERR_LAUNCH;
        if (flag & 1u) return KDA_ERR_DECAY_BOUND;
    }
    hipError_t e = launch_decode_commit_kept(dtype == KDA_DTYPE_BF16 ? 1 : 0, k, g, u, n_accept, state, N, K, H, dk,
                                             dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_decode_commit_verify(const void *prev_k, const float *prev_g, const float *prev_u,
                             const int32_t *n_accept, int Kp, const void *q, const void *k, const void *v,
                             const float *g, const float *beta, float *state, void *o, float *u, int N, int K, int H,
                             int dk, int dv, kda_dtype dtype, unsigned flags, hipStream_t stream) {
    int st = decode_multi_shape(N, K, H, dk, dv, dtype);
    if (st != KDA_OK) return st;
    if (Kp < 0 || int64_t(N) * Kp * H > INT32_MAX) return KDA_ERR_SHAPE;
    if (N == 0 || (K == 0 && Kp == 0)) return KDA_OK;
    if (!state) return KDA_ERR_NULL;
    if (Kp > 0 && (!prev_k || !prev_g || !prev_u || !n_accept)) return KDA_ERR_NULL;
    if (K > 0 && (!q || !k || !v || !g || !beta || !o)) return KDA_ERR_NULL;
    const size_t eb = dtype_bytes(dtype), prows = size_t(N) * Kp * H, rows = size_t(N) * K * H;
    const size_t nstate = size_t(N) * H * dk * dv * 4, no = rows * dv * eb, nu = rows * dv * 4;
    struct Buf { const void *p; size_t n; };
    const Buf ins[] = {{prev_k, prows * dk * eb}, {prev_g, prows * dk * 4}, {prev_u, prows * dv * 4},
                       {n_accept, size_t(N) * 4}, {q, rows * dk * eb}, {k, rows * dk * eb}, {v, rows * dv * eb},
                       {g, rows * dk * 4}, {beta, rows * 4}};
    for (const Buf &b : ins) {
        if (!b.p || b.n == 0) continue;
        if (misaligned(b.p, b.p == n_accept ? 4 : 16)) return KDA_ERR_ALIGN;
        if (overlap(state, nstate, b.p, b.n) || overlap(o, no, b.p, b.n) || overlap(u, nu, b.p, b.n))
            return KDA_ERR_ALIAS;
    }
    if (misaligned(state, 16) || misaligned(o, 16) || misaligned(u, 16)) return KDA_ERR_ALIGN;
    if (overlap(state, nstate, o, no) || overlap(state, nstate, u, nu) || overlap(o, no, u, nu)) return KDA_ERR_ALIAS;
    if (flags & KDA_FLAG_CHECK_DECAY) {  // both rounds' decays (each check reports its own flag)
        unsigned fp = 0, fn = 0;
        if (prows && run_checks(prev_g, prows * dk, nullptr, 0, 0, nullptr, stream, &fp) != hipSuccess)
            return KDA_ERR_LAUNCH;
        if (rows && run_checks(g, rows * dk, nullptr, 0, 0, nullptr, stream, &fn) != hipSuccess)
            return KDA_ERR_LAUNCH;
        if ((fp | fn) & 1u) return KDA_ERR_DECAY_BOUND;
    }
    const int dt = dtype == KDA_DTYPE_BF16 ? 1 : 0;
    hipError_t e = (K == 0) ? launch_decode_commit_kept(dt, prev_k, prev_g, prev_u, n_accept, state, N, Kp, H, dk,
                                                        dv, stream)
                            : launch_decode_commit_verify(dt, prev_k, prev_g, prev_u, n_accept, Kp, q, k, v, g, beta,
                                                          state, o, u, N, K, H, dk, dv, stream);
    return e == hipSuccess ? KDA_OK : KDA_ERR_LAUNCH;
}

int kda_profile_start(int max_launches) {
    if (max_launches <= 0) return KDA_ERR_SHAPE;
    if (g_prof.active) return KDA_ERR_SHAPE;
    for (hipEvent_t e : g_prof.evs) (void)hipEventDestroy(e);
    g_prof.evs.assign(2 * size_t(max_launches), nullptr);
    // timing-only events: without the system-scope fence an event record
    // costs no cache write-back between the launches it brackets
    for (auto &e : g_prof.evs)
        if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return KDA_ERR_LAUNCH;
    g_prof.names.assign(size_t(max_launches), std::string());
    g_prof.cap = max_launches;
    g_prof.used = 0;
    g_prof.active = true;
    return KDA_OK;
}

int kda_profile_stop(kda_kernel_time *out, int max_entries, int *n_entries) {
    if (!g_prof.active) return KDA_ERR_SHAPE;
    g_prof.active = false;
    std::vector<kda_kernel_time> agg;
    int status = KDA_OK;
    for (int i = 0; i < g_prof.used; ++i) {
        if (hipEventSynchronize(g_prof.evs[2 * i + 1]) != hipSuccess) { status = KDA_ERR_LAUNCH; break; }
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, g_prof.evs[2 * i], g_prof.evs[2 * i + 1]) != hipSuccess) {
            status = KDA_ERR_LAUNCH;
            break;
        }
        auto it = std::find_if(agg.begin(), agg.end(),
                               [&](const kda_kernel_time &t) { return g_prof.names[i] == t.name; });
        if (it == agg.end()) {
            kda_kernel_time t;
            memset(&t, 0, sizeof(t));
            strncpy(t.name, g_prof.names[i].c_str(), sizeof(t.name) - 1);
            agg.push_back(t);
            it = agg.end() - 1;
        }
        it->launches += 1;
        it->total_ms += ms;
    }
    for (hipEvent_t e : g_prof.evs) (void)hipEventDestroy(e);
    g_prof.evs.clear();
    g_prof.used = 0;
    g_prof.cap = 0;
    const int n = std::min<int>(int(agg.size()), std::max(max_entries, 0));
    for (int i = 0; i < n; ++i) out[i] = agg[i];
    if (n_entries) *n_entries = int(agg.size());
    return status;
}

}  // extern "C"
