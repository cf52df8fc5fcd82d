// Small support kernels: the packed-batch chunk map and the debug checks.
#include "kda_device.h"
#include "kda_launch.h"

namespace kda {

// coff[n] = first chunk slot of sequence n = sum over m < n of
// ceil(len_m / C), clamped to the workspace's nc_max slots; with ck_tokens
// > 0 also ckoff[n] = sum over m < n of floor(len_m / ck_tokens), the first
// checkpoint of sequence n.  Lengths come from cu_seqlens clamped to
// [0, T], so malformed offsets can never produce an out-of-range slot.  One
// workgroup; sequences in tiles of 1024.
__global__ __launch_bounds__(1024) void kda_chunk_offsets_kernel(const int32_t *__restrict__ cu, int N, int T,
                                                                 int C, int nc_max, int32_t *__restrict__ coff,
                                                                 int ck_tokens, int32_t *__restrict__ ckoff) {
    __shared__ int32_t scan[2][1024];
    __shared__ int32_t carry[2];
    const int tid = threadIdx.x;
    const bool ck = ck_tokens > 0;
    if (tid == 0) {
        carry[0] = carry[1] = 0;
        coff[0] = 0;
        if (ck) ckoff[0] = 0;
    }
    __syncthreads();
    for (int base = 0; base < N; base += 1024) {
        const int n = base + tid;
        int cnt = 0, nck = 0;
        if (n < N) {
            int s = cu[n], e = cu[n + 1];
            s = s < 0 ? 0 : (s > T ? T : s);
            e = e < s ? s : (e > T ? T : e);
            cnt = (e - s + C - 1) / C;
            nck = ck ? (e - s) / ck_tokens : 0;
        }
        scan[0][tid] = cnt;
        scan[1][tid] = nck;
        __syncthreads();
        for (int off = 1; off < 1024; off <<= 1) {
            const int x0 = (tid >= off) ? scan[0][tid - off] : 0;
            const int x1 = (tid >= off) ? scan[1][tid - off] : 0;
            __syncthreads();
            scan[0][tid] += x0;
            scan[1][tid] += x1;
            __syncthreads();
        }
        if (n < N) {
            coff[n + 1] = min(carry[0] + scan[0][tid], nc_max);
            if (ck) ckoff[n + 1] = carry[1] + scan[1][tid];
        }
        __syncthreads();
        if (tid == 1023) {
            carry[0] = min(carry[0] + scan[0][1023], nc_max);
            carry[1] = carry[1] + scan[1][1023];
        }
        __syncthreads();
    }
}

hipError_t launch_chunk_offsets(const int32_t *cu, int N, int T, int C, int nc_max, int32_t *coff, int ck_tokens,
                                int32_t *ckoff, hipStream_t s) {
    prof_begin(s);
    hipLaunchKernelGGL(kda_chunk_offsets_kernel, dim3(1), dim3(1024), 0, s, cu, N, T, C, nc_max, coff, ck_tokens,
                       ckoff);
    prof_end(s, "kda_chunk_offsets");
    return hipGetLastError();
}

// ---- debug checks (KDA_FLAG_CHECK_DECAY) ----
// The result word lives where the caller says: the prefill passes a word of
// its own workspace, so checked prefills on different streams never share
// it; the decode calls (which take no workspace) share this one per device.
__device__ unsigned int g_kda_check_flag;

__global__ void kda_flag_reset_kernel(unsigned *flag) { *flag = 0u; }

__global__ void kda_check_decay_kernel(const float *__restrict__ g, size_t n, unsigned *flag) {
    unsigned bad = 0;
    const size_t stride = size_t(gridDim.x) * blockDim.x;
    for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = g[i];
        if (!(x >= -5.f && x <= 0.f)) bad = 1u;  // NaN fails both comparisons
    }
    if (bad) atomicOr(flag, 1u);
}

__global__ void kda_check_cu_kernel(const int32_t *__restrict__ cu, int N, int T, unsigned *flag) {
    unsigned bad = 0;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < N; i += gridDim.x * blockDim.x)
        if (cu[i + 1] < cu[i]) bad = 2u;
    if (blockIdx.x == 0 && threadIdx.x == 0 && (cu[0] != 0 || cu[N] != T)) bad = 2u;
    if (bad) atomicOr(flag, bad);
}

hipError_t run_checks(const float *g, size_t n, const int32_t *cu, int N, int T, unsigned *flag_dev, hipStream_t s,
                      unsigned *flag_out) {
    if (!flag_dev) {
        hipError_t e = hipGetSymbolAddress(reinterpret_cast<void **>(&flag_dev), HIP_SYMBOL(g_kda_check_flag));
        if (e != hipSuccess) return e;
    }
    // a fill kernel, not a memset node: safe inside a captured graph
    hipLaunchKernelGGL(kda_flag_reset_kernel, dim3(1), dim3(1), 0, s, flag_dev);
    if (n > 0) {
        size_t blocks = (n + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(kda_check_decay_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, g, n, flag_dev);
    }
    if (cu) {
        const int blocks = N / 256 + 1 > 1024 ? 1024 : N / 256 + 1;
        hipLaunchKernelGGL(kda_check_cu_kernel, dim3(blocks), dim3(256), 0, s, cu, N, T, flag_dev);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    unsigned flag = 0;
    e = hipMemcpyAsync(&flag, flag_dev, sizeof(flag), hipMemcpyDeviceToHost, s);
    if (e != hipSuccess) return e;
    e = hipStreamSynchronize(s);
    if (e != hipSuccess) return e;
    *flag_out = flag;
    return hipSuccess;
}

}  // namespace kda
