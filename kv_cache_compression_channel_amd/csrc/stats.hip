// stats.hip -- quantization error statistics (Walkthrough (KV Compression 公式到源码对照) §1.3:
// RMSE, max_abs_error, mean_abs_error) and the kvq_dequant dispatcher.
//
// Two-stage deterministic reduction: a fixed number of blocks each reduce one fixed
// contiguous chunk (fp64 differences, squares and absolute values), then one block adds
// the partials in a fixed tree order.  No atomics, so results repeat bit for bit.
#include "kvq_internal.h"

namespace kvq {

int dequant_pc(const kvq_pc_tensor* t, void* out, int ot, hipStream_t st);
int dequant_int4(const kvq_int4_cache* c, bool is_k, void* out, int ot, hipStream_t st);

namespace {

constexpr int kThreads = 256;
constexpr int kBlocks = 2048;

template <int XT, int VEC>
__device__ __forceinline__ void ld(const void* p, int64_t i, double (&v)[VEC]) {
    if constexpr (XT == KVQ_FP32) {
        const float* f = static_cast<const float*>(p) + i;
        if constexpr (VEC == 8) {
            const float4 a = ld_stream_f4(f);
            const float4 b = ld_stream_f4(f + 4);
            v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        } else {
            v[0] = *f;
        }
    } else {
        const uint16_t* h = static_cast<const uint16_t*>(p) + i;
        if constexpr (VEC == 8) {
            const uint4 a = ld_stream_u4(h);
            v[0] = bf_lo(a.x); v[1] = bf_hi(a.x); v[2] = bf_lo(a.y); v[3] = bf_hi(a.y);
            v[4] = bf_lo(a.z); v[5] = bf_hi(a.z); v[6] = bf_lo(a.w); v[7] = bf_hi(a.w);
        } else {
            v[0] = bf_to_f(*h);
        }
    }
}

__device__ __forceinline__ void block_reduce3(double& a, double& b, double& c, double* sh) {
#pragma unroll
    for (int off = 32; off >= 1; off /= 2) {
        a += __shfl_xor(a, off);
        b += __shfl_xor(b, off);
        c = fmax(c, __shfl_xor(c, off));
    }
    const int w = threadIdx.x / 64;
    if (threadIdx.x % 64 == 0) { sh[3 * w] = a; sh[3 * w + 1] = b; sh[3 * w + 2] = c; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; ++i) { a += sh[3 * i]; b += sh[3 * i + 1]; c = fmax(c, sh[3 * i + 2]); }
    }
}

template <int XT, int HT, int VEC>
__global__ void __launch_bounds__(kThreads) stats_partial_kernel(const void* __restrict__ x, const void* __restrict__ xh,
                                                                 int64_t n, int64_t chunk, double* __restrict__ part) {
    __shared__ double sh[3 * (kThreads / 64)];
    const int64_t lo = (int64_t)blockIdx.x * chunk, hi = min(n, lo + chunk);
    double sq = 0.0, ab = 0.0, mx = 0.0;
    auto acc = [&](const double (&a)[VEC], const double (&b)[VEC]) {
#pragma unroll
        for (int k = 0; k < VEC; ++k) {
            const double e = a[k] - b[k];
            sq = __builtin_fma(e, e, sq);
            ab += __builtin_fabs(e);
            mx = __builtin_fmax(mx, __builtin_fabs(e));
        }
    };
    constexpr int64_t step = (int64_t)kThreads * VEC;
    int64_t i = lo + (int64_t)threadIdx.x * VEC;
    for (; i + step < hi; i += 2 * step) {   // two independent load pairs in flight
        double a0[VEC], b0[VEC], a1[VEC], b1[VEC];
        ld<XT, VEC>(x, i, a0);
        ld<HT, VEC>(xh, i, b0);
        ld<XT, VEC>(x, i + step, a1);
        ld<HT, VEC>(xh, i + step, b1);
        acc(a0, b0);
        acc(a1, b1);
    }
    if (i < hi) {
        double a0[VEC], b0[VEC];
        ld<XT, VEC>(x, i, a0);
        ld<HT, VEC>(xh, i, b0);
        acc(a0, b0);
    }
    block_reduce3(sq, ab, mx, sh);
    if (threadIdx.x == 0) {
        part[3 * blockIdx.x] = sq;
        part[3 * blockIdx.x + 1] = ab;
        part[3 * blockIdx.x + 2] = mx;
    }
}

__global__ void __launch_bounds__(kThreads) stats_final_kernel(const double* __restrict__ part, int nblk,
                                                               double* __restrict__ out) {
    __shared__ double sh[3 * (kThreads / 64)];
    double sq = 0.0, ab = 0.0, mx = 0.0;
    for (int i = threadIdx.x; i < nblk; i += kThreads) {
        sq += part[3 * i];
        ab += part[3 * i + 1];
        mx = fmax(mx, part[3 * i + 2]);
    }
    block_reduce3(sq, ab, mx, sh);
    if (threadIdx.x == 0) { out[0] = sq; out[1] = ab; out[2] = mx; }
}

template <int XT, int HT>
void launch_stats(const void* x, const void* xh, int64_t n, bool vec8, double* out, double* part, hipStream_t st) {
    const int64_t step = (int64_t)kThreads * 8;
    const int64_t chunk = cdiv(cdiv(n, kBlocks), step) * step;
    const int nblk = (int)cdiv(n, chunk);
    if (vec8)
        hipLaunchKernelGGL((stats_partial_kernel<XT, HT, 8>), dim3(nblk), dim3(kThreads), 0, st, x, xh, n, chunk, part);
    else
        hipLaunchKernelGGL((stats_partial_kernel<XT, HT, 1>), dim3(nblk), dim3(kThreads), 0, st, x, xh, n, chunk, part);
    hipLaunchKernelGGL(stats_final_kernel, dim3(1), dim3(kThreads), 0, st, part, nblk, out);
}

}  // namespace
}  // namespace kvq

extern "C" {

size_t kvq_err_stats_ws(int64_t n) {
    if (n < 1) return 0;
    return (size_t)kvq::kBlocks * 3 * sizeof(double);
}

int kvq_err_stats(const void* x, int xt, const void* xhat, int ht, int64_t n, double* dev_out, void* ws,
                  size_t ws_bytes, kvq_stream stream) {
    KVQ_REQUIRE(x && xhat && dev_out, "kvq_err_stats: NULL pointer");
    KVQ_REQUIRE(n >= 1, "kvq_err_stats: n must be >= 1");
    KVQ_REQUIRE((xt == KVQ_FP32 || xt == KVQ_BF16) && (ht == KVQ_FP32 || ht == KVQ_BF16),
                "kvq_err_stats: dtypes must be KVQ_FP32 or KVQ_BF16");
    KVQ_REQUIRE(ws && ws_bytes >= kvq_err_stats_ws(n), "kvq_err_stats: workspace of %zu bytes needed",
                kvq_err_stats_ws(n));
    KVQ_REQUIRE_ALIGNED(x, "x");
    KVQ_REQUIRE_ALIGNED(xhat, "xhat");
    KVQ_REQUIRE((reinterpret_cast<uintptr_t>(dev_out) & 7u) == 0, "kvq_err_stats: dev_out must be 8-byte aligned");
    KVQ_REQUIRE_ALIGNED(ws, "ws");
    hipStream_t st = static_cast<hipStream_t>(stream);
    const bool vec8 = n % 8 == 0;
    double* part = static_cast<double*>(ws);
    if (xt == KVQ_FP32 && ht == KVQ_FP32) kvq::launch_stats<KVQ_FP32, KVQ_FP32>(x, xhat, n, vec8, dev_out, part, st);
    else if (xt == KVQ_FP32) kvq::launch_stats<KVQ_FP32, KVQ_BF16>(x, xhat, n, vec8, dev_out, part, st);
    else if (ht == KVQ_FP32) kvq::launch_stats<KVQ_BF16, KVQ_FP32>(x, xhat, n, vec8, dev_out, part, st);
    else kvq::launch_stats<KVQ_BF16, KVQ_BF16>(x, xhat, n, vec8, dev_out, part, st);
    return kvq::launch_status("kvq_err_stats");
}

int kvq_dequant(const kvq_qdesc* src, void* out, int ot, kvq_stream stream) {
    KVQ_REQUIRE(src && src->desc, "kvq_dequant: NULL descriptor");
    hipStream_t st = static_cast<hipStream_t>(stream);
    switch (src->kind) {
        case KVQ_FMT_PER_CHANNEL:
            return kvq::dequant_pc(static_cast<const kvq_pc_tensor*>(src->desc), out, ot, st);
        case KVQ_FMT_INT4_K:
            return kvq::dequant_int4(static_cast<const kvq_int4_cache*>(src->desc), true, out, ot, st);
        case KVQ_FMT_INT4_V:
            return kvq::dequant_int4(static_cast<const kvq_int4_cache*>(src->desc), false, out, ot, st);
        default:
            return kvq::fail(KVQ_EINVAL, "kvq_dequant: unknown kind %d", src->kind);
    }
}

}  // extern "C"
