// host_common.hip -- error state, launch checks and the host-only accounting helpers.
#include <cmath>
#include <cstdarg>

#include "kvq_internal.h"

namespace kvq {

static thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

void clear_error() { g_last_error.clear(); }

int launch_status(const char* what) {
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(KVQ_EHIP, "%s: %s", what, hipGetErrorString(e));
    return KVQ_OK;
}

}  // namespace kvq

extern "C" {

const char* kvq_last_error(void) { return kvq::g_last_error.c_str(); }

int kvq_abi_version(void) { return 1; }

int kvq_stats_finalize(const double in[3], int64_t n, double* rmse, double* max_abs, double* mean_abs) {
    KVQ_REQUIRE(in && rmse && max_abs && mean_abs, "kvq_stats_finalize: NULL pointer");
    KVQ_REQUIRE(n >= 1, "kvq_stats_finalize: n must be >= 1 (got %lld)", (long long)n);
    *rmse = std::sqrt(in[0] / (double)n);
    *max_abs = in[2];
    *mean_abs = in[1] / (double)n;
    return KVQ_OK;
}

double kvq_compression_ratio(uint64_t orig_bytes, uint64_t data, uint64_t scale, uint64_t zp) {
    const uint64_t den = data + scale + zp;
    return den ? (double)orig_bytes / (double)den : 0.0;
}

uint64_t kvq_int4_bytes(uint64_t N, uint64_t g) {
    if (g == 0) return 0;
    return N / 2 + (N & 1) + (N / g + (N % g != 0)) * 4;
}

int kvq_token_ratio(int64_t T, int64_t K, double* out) {
    KVQ_REQUIRE(out, "kvq_token_ratio: NULL out");
    KVQ_REQUIRE(T > 0 && K > 0 && K <= T, "kvq_token_ratio: require 0 < kept (%lld) <= total (%lld)",
                (long long)K, (long long)T);
    *out = (double)T / (double)K;
    return KVQ_OK;
}

int kvq_total_gain(double s_old, double s_new, int64_t T, int64_t K, double* out) {
    KVQ_REQUIRE(out, "kvq_total_gain: NULL out");
    KVQ_REQUIRE(T > 0 && K > 0 && K <= T, "kvq_total_gain: require 0 < kept <= total");
    KVQ_REQUIRE(s_new > 0.0, "kvq_total_gain: s_new must be > 0");
    *out = (s_old / s_new) * ((double)T / (double)K);
    return KVQ_OK;
}

uint64_t kvq_kv_bytes(uint64_t L, uint64_t T, uint64_t C, uint64_t b, uint64_t metadata) {
    return L * T * C * b + metadata;
}

int64_t kvq_keep_count(int64_t T, int64_t budget, int64_t window) {
    if (T < 1 || budget < 0 || window < 0) return -1;
    const int64_t recent = window < T ? window : T;
    const int64_t k = budget > recent ? budget : recent;
    return k < T ? k : T;
}

}  // extern "C"
