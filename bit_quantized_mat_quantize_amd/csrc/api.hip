// api.hip -- the extern "C" entry points of libqmm (declared in include/qmm.h).
//
// Every entry point validates its arguments on the host before touching the
// HIP runtime, so a bad call returns an error code, enqueues nothing and needs
// no GPU to be tested.  Valid calls dispatch to the kernel families in
// quantize.hip, repack.hip, gemv.hip, skinny.hip, gemm.hip, q6k.hip,
// q6k_gemm.hip, q2k.hip, q2k_gemm.hip, q40_gemm.hip and moe.hip.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>

#include "../../include/qmm.h"
#include "qmm_launch.h"

namespace {

thread_local char g_err[512] = "";

qmm_status fail(qmm_status st, const char *fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

constexpr int64_t kMaxRows = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 20;
// Q4_K small batches of at most this many rows take the 16 x 16-tile kernel
// (skinny16.hip): from 3 to 16 rows it was as fast as the 32 x 32 kernel or
// faster on every shape measured (N = 4096 .. 28672, K = 4096 .. 14336), up
// to 1.6x where N / 32 is below the CU count.
constexpr int64_t kSkinny16MaxM = 16;

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int act_qk(qmm_act_type t) { return t == QMM_Q8_0 ? 32 : (t == QMM_Q8_K ? 256 : 0); }
int act_bytes_per_block(qmm_act_type t) { return t == QMM_Q8_0 ? 34 : 292; }
int w_qk(qmm_weight_type t) {
    return t == QMM_Q4_0 ? 32 : ((t == QMM_Q4_K || t == QMM_Q6_K || t == QMM_Q2_K) ? 256 : 0);
}
int w_bytes_per_block(qmm_weight_type t) {
    return t == QMM_Q4_0 ? 18 : (t == QMM_Q6_K ? 210 : (t == QMM_Q2_K ? 84 : 144));
}

// The MFMA kernels address the weight and the activation matrix with 32-bit
// buffer offsets.
bool below_4gib(qmm_weight_type t, qmm_layout l, int64_t M, int64_t N, int64_t K) {
    const size_t lim = size_t(1) << 32;
    const qmm_act_type at = t == QMM_Q4_0 ? QMM_Q8_0 : QMM_Q8_K;
    return qmm_weight_bytes(t, l, N, K) < lim && qmm_act_bytes(at, M, K) < lim;
}

qmm_status check_rows(const char *name, int64_t v) {
    if (v < 0) return fail(QMM_EINVAL, "%s = %lld is negative", name, (long long)v);
    if (v > kMaxRows)
        return fail(QMM_EUNSUPPORTED, "%s = %lld exceeds the limit %lld", name, (long long)v,
                    (long long)kMaxRows);
    return QMM_OK;
}

qmm_status check_k(int64_t K, int qk) {
    if (K <= 0 || K % qk != 0)
        return fail(QMM_EUNSUPPORTED, "K = %lld must be a positive multiple of %d", (long long)K, qk);
    if (K > kMaxK)
        return fail(QMM_EUNSUPPORTED, "K = %lld exceeds the limit %lld", (long long)K, (long long)kMaxK);
    return QMM_OK;
}

qmm_status check_ptr(const char *name, const void *p) {
    if (!p) return fail(QMM_EINVAL, "%s is NULL", name);
    if (!aligned16(p)) return fail(QMM_EALIGN, "%s = %p is not 16-byte aligned", name, p);
    return QMM_OK;
}

qmm_status check_size(const char *name, size_t have, size_t need) {
    if (have < need)
        return fail(QMM_EINVAL, "%s holds %zu bytes, %zu needed", name, have, need);
    return QMM_OK;
}

qmm_status device_status(hipError_t e, const char *what) {
    if (e == hipSuccess) return QMM_OK;
    return fail(QMM_EDEVICE, "%s: %s", what, hipGetErrorString(e));
}

// QMM_LOG set to anything but "" or "0" prints every mul_mat call's kernel
// choice, with its output tile, to stderr (read once per process).
bool log_enabled() {
    static const bool on = [] {
        const char *v = getenv("QMM_LOG");
        return v != nullptr && v[0] != '\0' && !(v[0] == '0' && v[1] == '\0');
    }();
    return on;
}

const char *algo_name(qmm_algo a) {
    switch (a) {
        case QMM_ALGO_AUTO: return "AUTO";
        case QMM_ALGO_GEMV: return "GEMV";
        case QMM_ALGO_MFMA: return "MFMA";
        case QMM_ALGO_SKINNY: return "SKINNY";
    }
    return "?";
}

const char *family_tile(qmm_algo a) {
    switch (a) {
        case QMM_ALGO_GEMV: return "one wavefront per output row, up to 8 activation rows per launch";
        case QMM_ALGO_SKINNY:
            return "small-batch MFMA kernel: 16 or 32 columns per workgroup, K split inside the workgroup, "
                   "weights read once per 32-row chunk";
        case QMM_ALGO_MFMA: return "128 x 256 output tile per workgroup";
        default: return "";
    }
}

void log_choice(const char *entry, const char *fmt, qmm_layout l, int64_t M, int64_t N, int64_t K,
                qmm_algo asked, qmm_algo taken) {
    if (!log_enabled()) return;
    fprintf(stderr, "qmm: %s %s M=%lld N=%lld K=%lld layout=%s algo=%s -> %s (%s)\n", entry, fmt,
            (long long)M, (long long)N, (long long)K, l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical",
            algo_name(asked), algo_name(taken), family_tile(taken));
}

#define QMM_TRY(expr)                        \
    do {                                     \
        const qmm_status st_ = (expr);       \
        if (st_ != QMM_OK) return st_;       \
    } while (0)

qmm_status mul_mat_common(qmm_weight_type wt, const void *w, size_t w_bytes, qmm_layout l,
                          const void *y, size_t y_bytes, const float *out, size_t out_bytes,
                          int64_t M, int64_t N, int64_t K) {
    if (l != QMM_LAYOUT_CANONICAL && l != QMM_LAYOUT_REPACKED)
        return fail(QMM_EUNSUPPORTED, "unknown layout %d", (int)l);
    QMM_TRY(check_rows("M", M));
    QMM_TRY(check_rows("N", N));
    QMM_TRY(check_k(K, w_qk(wt)));
    if (M == 0 || N == 0) return QMM_OK;
    QMM_TRY(check_ptr("w", w));
    QMM_TRY(check_ptr("y", y));
    QMM_TRY(check_ptr("out", out));
    QMM_TRY(check_size("w", w_bytes, qmm_weight_bytes(wt, l, N, K)));
    const qmm_act_type at = wt == QMM_Q4_0 ? QMM_Q8_0 : QMM_Q8_K;
    QMM_TRY(check_size("y", y_bytes, qmm_act_bytes(at, M, K)));
    QMM_TRY(check_size("out", out_bytes, (size_t)(M * N) * sizeof(float)));
    return QMM_OK;
}

}  // namespace

extern "C" {

size_t qmm_act_bytes(qmm_act_type t, int64_t M, int64_t K) {
    const int qk = act_qk(t);
    if (!qk || M < 0 || K < 0 || K % qk) return 0;
    return (size_t)(M * (K / qk) * act_bytes_per_block(t));
}

size_t qmm_weight_bytes(qmm_weight_type t, qmm_layout l, int64_t N, int64_t K) {
    const int qk = w_qk(t);
    if (!qk || N < 0 || K < 0 || K % qk) return 0;
    if (l != QMM_LAYOUT_CANONICAL && l != QMM_LAYOUT_REPACKED) return 0;
    if (t == QMM_Q4_0 && l == QMM_LAYOUT_REPACKED) return (size_t)qmm::repacked_bytes_q4_0(N, K);
    if (t == QMM_Q6_K && l == QMM_LAYOUT_REPACKED) return (size_t)qmm::repacked_bytes_q6_K(N, K);
    if (t == QMM_Q2_K && l == QMM_LAYOUT_REPACKED) return (size_t)qmm::repacked_bytes_q2_K(N, K);
    return (size_t)(N * (K / qk) * w_bytes_per_block(t));
}

qmm_status qmm_quantize_row_q8(qmm_act_type t, const float *x, int64_t M, int64_t K, void *y,
                               size_t y_bytes, void *stream) {
    const int qk = act_qk(t);
    if (!qk) return fail(QMM_EUNSUPPORTED, "unknown activation type %d", (int)t);
    QMM_TRY(check_rows("M", M));
    QMM_TRY(check_k(K, qk));
    if (M == 0) return QMM_OK;
    QMM_TRY(check_ptr("x", x));
    QMM_TRY(check_ptr("y", y));
    QMM_TRY(check_size("y", y_bytes, qmm_act_bytes(t, M, K)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *yo = static_cast<uint8_t *>(y);
    return device_status(t == QMM_Q8_K ? qmm::launch_quantize_q8_K(x, yo, M, K, s)
                                       : qmm::launch_quantize_q8_0(x, yo, M, K, s),
                         "quantize_row_q8 launch");
}

qmm_status qmm_quantize_weights(qmm_weight_type t, const float *w, int64_t N, int64_t K, void *out,
                                size_t out_bytes, void *stream) {
    const int qk = w_qk(t);
    if (!qk) return fail(QMM_EUNSUPPORTED, "unknown weight type %d", (int)t);
    QMM_TRY(check_rows("N", N));
    QMM_TRY(check_k(K, qk));
    if (N == 0) return QMM_OK;
    QMM_TRY(check_ptr("w", w));
    QMM_TRY(check_ptr("out", out));
    QMM_TRY(check_size("out", out_bytes, qmm_weight_bytes(t, QMM_LAYOUT_CANONICAL, N, K)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *o = static_cast<uint8_t *>(out);
    return device_status(t == QMM_Q4_K   ? qmm::launch_encode_q4_K(w, o, N, K, s)
                         : t == QMM_Q6_K ? qmm::launch_encode_q6_K(w, o, N, K, s)
                         : t == QMM_Q2_K ? qmm::launch_encode_q2_K(w, o, N, K, s)
                                         : qmm::launch_encode_q4_0(w, o, N, K, s),
                         "quantize_weights launch");
}

qmm_status qmm_repack_weights(qmm_weight_type t, const void *w_canon, int64_t N, int64_t K,
                              void *w_repacked, size_t out_bytes, void *stream) {
    const int qk = w_qk(t);
    if (!qk) return fail(QMM_EUNSUPPORTED, "unknown weight type %d", (int)t);
    QMM_TRY(check_rows("N", N));
    QMM_TRY(check_k(K, qk));
    if (N == 0) return QMM_OK;
    QMM_TRY(check_ptr("w_canon", w_canon));
    QMM_TRY(check_ptr("w_repacked", w_repacked));
    const size_t need = qmm_weight_bytes(t, QMM_LAYOUT_REPACKED, N, K);
    QMM_TRY(check_size("w_repacked", out_bytes, need));
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(w_canon);
    const uintptr_t b0 = reinterpret_cast<uintptr_t>(w_repacked);
    const size_t in_bytes = qmm_weight_bytes(t, QMM_LAYOUT_CANONICAL, N, K);
    if (a0 < b0 + need && b0 < a0 + in_bytes)
        return fail(QMM_EINVAL, "w_canon and w_repacked overlap");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *in = static_cast<const uint8_t *>(w_canon);
    uint8_t *o = static_cast<uint8_t *>(w_repacked);
    return device_status(t == QMM_Q4_K   ? qmm::launch_repack_q4_K(in, o, N, K, s)
                         : t == QMM_Q6_K ? qmm::launch_repack_q6_K(in, o, N, K, s)
                         : t == QMM_Q2_K ? qmm::launch_repack_q2_K(in, o, N, K, s)
                                         : qmm::launch_repack_q4_0(in, o, N, K, s),
                         "repack_weights launch");
}

// Q4_0 small-batch kernel vs GEMM: its time grows with the number of 32-row
// chunks times N/32 workgroups, the GEMM's stays one K loop while its row
// tiles fit the CUs; measured on N = 4096..28672, K = 4096..14336 it wins
// while ceil(M/32)*N stays at or below this.
constexpr int64_t kSkinnyMN_Q4_0 = 16 * 8192;

qmm_status qmm_mul_mat_q4_0_ex(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                               size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                               int64_t K, qmm_algo algo, void *stream) {
    if (algo != QMM_ALGO_AUTO && algo != QMM_ALGO_GEMV && algo != QMM_ALGO_MFMA && algo != QMM_ALGO_SKINNY)
        return fail(QMM_EUNSUPPORTED, "unknown algo %d", (int)algo);
    QMM_TRY(mul_mat_common(QMM_Q4_0, w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K));
    // the MFMA kernels step K by 256 and take the repacked layout
    const bool mfma_ok = l == QMM_LAYOUT_REPACKED && K % 256 == 0 && below_4gib(QMM_Q4_0, l, M, N, K);
    const bool skinny_ok = mfma_ok && M <= qmm::skinny_q4_0_max_m();
    if (algo == QMM_ALGO_MFMA && !mfma_ok)
        return fail(QMM_EUNSUPPORTED,
                    "Q4_0 MFMA path takes the repacked layout, K a multiple of 256 and matrices below 4 GiB");
    if (algo == QMM_ALGO_SKINNY && !skinny_ok)
        return fail(QMM_EUNSUPPORTED,
                    "Q4_0 SKINNY path takes the repacked layout, K a multiple of 256, M <= %lld and matrices "
                    "below 4 GiB", (long long)qmm::skinny_q4_0_max_m());
    if (M == 0 || N == 0) return QMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const uint8_t *yb = static_cast<const uint8_t *>(y);
    qmm_algo a = algo;
    if (a == QMM_ALGO_AUTO) {
        // GEMV for M = 1; while the GEMV stages the rows in LDS, up to M = 4
        // (its pass over the weights per row is still cheaper than the
        // small-batch kernel: 18 against 21 us at M = 4, N = K = 8192) and up
        // to M*N = 36864 (N < 8192, where the small-batch kernel's N/32
        // workgroups leave CUs idle: 9.5 against 12.1 us at M = 8, N = 4096);
        // for M = 2 below 8192 columns; and where the MFMA kernels are ruled out
        if (!mfma_ok || M == 1 || (qmm::gemv_q4_0s_fits(M, K) && (M <= 4 || M * N <= 36864)) ||
            (M == 2 && N < 8192))
            a = QMM_ALGO_GEMV;
        else if (skinny_ok && ((M + 31) / 32) * N <= kSkinnyMN_Q4_0) a = QMM_ALGO_SKINNY;
        else a = QMM_ALGO_MFMA;
    }
    log_choice("mul_mat", "Q4_0", l, M, N, K, algo, a);
    if (a == QMM_ALGO_SKINNY)
        return device_status(qmm::launch_skinny_q4_0(wb, (int64_t)qmm_weight_bytes(QMM_Q4_0, l, N, K), yb, out,
                                                     M, N, K, s),
                             "mul_mat_q4_0 small-batch launch");
    if (a == QMM_ALGO_MFMA)
        return device_status(qmm::launch_gemm_q4_0(wb, (int64_t)qmm_weight_bytes(QMM_Q4_0, l, N, K), yb,
                                                   out, M, N, K, s),
                             "mul_mat_q4_0 gemm launch");
    // groups of up to 8 activation rows per GEMV launch
    const bool rep = l == QMM_LAYOUT_REPACKED;
    for (int64_t m0 = 0; m0 < M; m0 += qmm::kGemvMaxM) {
        const int64_t mm = M - m0 < qmm::kGemvMaxM ? M - m0 : qmm::kGemvMaxM;
        QMM_TRY(device_status(qmm::launch_gemv_q4_0(wb, rep, yb + m0 * (K / 32) * 34, out + m0 * N,
                                                    mm, N, K, s),
                              "mul_mat_q4_0 gemv launch"));
    }
    return QMM_OK;
}

qmm_status qmm_mul_mat_q4_0(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                            size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                            int64_t K, void *stream) {
    return qmm_mul_mat_q4_0_ex(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, QMM_ALGO_AUTO,
                               stream);
}

qmm_status qmm_mul_mat_q4_K_ex(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                               size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                               int64_t K, qmm_algo algo, void *stream) {
    if (algo != QMM_ALGO_AUTO && algo != QMM_ALGO_GEMV && algo != QMM_ALGO_MFMA &&
        algo != QMM_ALGO_SKINNY)
        return fail(QMM_EUNSUPPORTED, "unknown algo %d", (int)algo);
    QMM_TRY(mul_mat_common(QMM_Q4_K, w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K));
    if (algo == QMM_ALGO_GEMV && M > qmm::kGemvMaxM)
        return fail(QMM_EUNSUPPORTED, "GEMV path takes M <= %d (M = %lld)", qmm::kGemvMaxM,
                    (long long)M);
    // the MFMA kernels address both matrices with 32-bit offsets
    const bool small = below_4gib(QMM_Q4_K, l, M, N, K);
    const bool skinny_ok = M <= qmm::skinny_max_m() && small;
    if (algo == QMM_ALGO_SKINNY && !skinny_ok)
        return fail(QMM_EUNSUPPORTED,
                    "SKINNY path takes M <= %lld and matrices below 4 GiB (M = %lld)",
                    (long long)qmm::skinny_max_m(), (long long)M);
    if (algo == QMM_ALGO_MFMA && !small)
        return fail(QMM_EUNSUPPORTED, "MFMA path takes matrices below 4 GiB");
    if (M == 0 || N == 0) return QMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool rep = l == QMM_LAYOUT_REPACKED;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const uint8_t *yb = static_cast<const uint8_t *>(y);
    qmm_algo a = algo;
    // AUTO: the small-batch kernels (K split over the wavefronts of a
    // workgroup; 16 x 16 tiles up to 16 rows, 32 x 32 above) beat the GEMM up
    // to 32 rows, and further while ceil(M/32)*N stays below 9*8192 (measured
    // at K = 8192: up to M ~ 300 for N = 8192, M ~ 80 for N = 28672); K
    // cancels, both scale with it.  From M = 2 on the 16 x 16 kernel is as
    // fast as the GEMV or faster (N = K = 4096: 5.6 against 6.3 us; N = 4096,
    // K = 14336: 11.6 against 17.2 us), whose vector work grows with M.
    if (a == QMM_ALGO_AUTO) {
        const bool skinny_pref = M <= 32 || ((M + 31) / 32) * N <= 9 * 8192;
        a = M == 1 ? QMM_ALGO_GEMV
                   : (skinny_ok && skinny_pref ? QMM_ALGO_SKINNY
                                               : (M <= qmm::kGemvMaxM || !small ? QMM_ALGO_GEMV : QMM_ALGO_MFMA));
    }
    log_choice("mul_mat", "Q4_K", l, M, N, K, algo, a);
    if (a == QMM_ALGO_GEMV) {
        // groups of up to 8 activation rows per GEMV launch
        const int64_t rowb = (K / 256) * 292;
        for (int64_t m0 = 0; m0 < M; m0 += qmm::kGemvMaxM) {
            const int64_t mm = M - m0 < qmm::kGemvMaxM ? M - m0 : qmm::kGemvMaxM;
            QMM_TRY(device_status(qmm::launch_gemv_q4_K(wb, rep, yb + m0 * rowb, out + m0 * N, mm, N, K, s),
                                  "mul_mat_q4_K gemv launch"));
        }
        return QMM_OK;
    }
    // the small-batch family: 16 x 16 tiles up to 16 rows, 32 x 32 above
    if (a == QMM_ALGO_SKINNY && M <= kSkinny16MaxM)
        return device_status(qmm::launch_skinny16_q4_K(wb, rep, yb, out, M, N, K, s),
                             "mul_mat_q4_K skinny launch");
    if (a == QMM_ALGO_SKINNY)
        return device_status(qmm::launch_skinny_q4_K(wb, rep, yb, out, M, N, K, s),
                             "mul_mat_q4_K skinny launch");
    return device_status(qmm::launch_gemm_q4_K(wb, rep, yb, out, M, N, K, s), "mul_mat_q4_K gemm launch");
}

qmm_status qmm_mul_mat_q4_K(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                            size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                            int64_t K, void *stream) {
    return qmm_mul_mat_q4_K_ex(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, QMM_ALGO_AUTO,
                               stream);
}

}  // extern "C"

namespace {

// Q6_K and Q2_K (16-element groups): a GEMV for any M while the activation
// row fits LDS; for the repacked layout also a small-batch kernel and an MFMA
// GEMM.
struct GroupedKernels {
    const char *name;
    int64_t gemv_max_k;
    hipError_t (*gemv)(const uint8_t *, bool, const uint8_t *, float *, int64_t, int64_t, int64_t,
                       hipStream_t);
    hipError_t (*gemm)(const uint8_t *, int64_t, const uint8_t *, float *, int64_t, int64_t, int64_t,
                       hipStream_t);
    // small-batch kernel (repacked layout), or null where the format has none;
    // AUTO takes it while ceil(M/32)*N <= skinny_mn
    hipError_t (*skinny)(const uint8_t *, int64_t, const uint8_t *, float *, int64_t, int64_t, int64_t,
                         hipStream_t);
    int64_t skinny_max_m, skinny_mn;
};

qmm_status mul_mat_grouped(qmm_weight_type t, const GroupedKernels &k, const void *w, size_t w_bytes,
                           qmm_layout l, const void *y, size_t y_bytes, float *out, size_t out_bytes,
                           int64_t M, int64_t N, int64_t K, qmm_algo algo, void *stream) {
    if (algo != QMM_ALGO_AUTO && algo != QMM_ALGO_GEMV && algo != QMM_ALGO_MFMA &&
        !(algo == QMM_ALGO_SKINNY && k.skinny))
        return fail(QMM_EUNSUPPORTED, "%s takes the GEMV%s or MFMA path (algo %d)", k.name,
                    k.skinny ? ", SKINNY" : "", (int)algo);
    QMM_TRY(mul_mat_common(t, w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K));
    const bool gemv_ok = K <= k.gemv_max_k;
    const bool mfma_ok = l == QMM_LAYOUT_REPACKED && below_4gib(t, l, M, N, K);
    const bool skinny_ok = k.skinny && mfma_ok && M <= k.skinny_max_m;
    if (algo == QMM_ALGO_SKINNY && !skinny_ok)
        return fail(QMM_EUNSUPPORTED, "%s SKINNY path takes the repacked layout, M <= %lld and matrices below 4 GiB",
                    k.name, (long long)k.skinny_max_m);
    if (algo == QMM_ALGO_GEMV && !gemv_ok)
        return fail(QMM_EUNSUPPORTED, "%s GEMV takes K <= %lld (K = %lld)", k.name,
                    (long long)k.gemv_max_k, (long long)K);
    if (algo == QMM_ALGO_MFMA && !mfma_ok)
        return fail(QMM_EUNSUPPORTED, "%s MFMA path takes the repacked layout and matrices below 4 GiB",
                    k.name);
    if (algo == QMM_ALGO_AUTO && !gemv_ok && !mfma_ok)
        return fail(QMM_EUNSUPPORTED,
                    "%s with K = %lld > %lld needs the repacked layout and matrices below 4 GiB", k.name,
                    (long long)K, (long long)k.gemv_max_k);
    if (M == 0 || N == 0) return QMM_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const uint8_t *yb = static_cast<const uint8_t *>(y);
    qmm_algo a = algo;
    if (a == QMM_ALGO_AUTO) {
        // the canonical layout (and a matrix of 4 GiB or more) has only the
        // GEMV; otherwise the GEMV for M = 1 and for M = 2 below 8192 columns
        // (fewer than 256 small-batch workgroups), the small-batch kernel
        // while its row chunks cost less than one GEMM K loop, the GEMM above.
        // A K past the GEMV's limit sends M = 1 and 2 down the same rule.
        if (!mfma_ok) a = QMM_ALGO_GEMV;
        else if ((M == 1 || (M == 2 && N < 8192)) && gemv_ok) a = QMM_ALGO_GEMV;
        else if (skinny_ok && ((M + 31) / 32) * N <= k.skinny_mn) a = QMM_ALGO_SKINNY;
        else a = QMM_ALGO_MFMA;
    }
    log_choice("mul_mat", k.name, l, M, N, K, algo, a);
    if (a == QMM_ALGO_GEMV)
        return device_status(k.gemv(wb, l == QMM_LAYOUT_REPACKED, yb, out, M, N, K, s), "mul_mat gemv launch");
    if (a == QMM_ALGO_SKINNY)
        return device_status(k.skinny(wb, (int64_t)qmm_weight_bytes(t, l, N, K), yb, out, M, N, K, s),
                             "mul_mat skinny launch");
    return device_status(k.gemm(wb, (int64_t)qmm_weight_bytes(t, l, N, K), yb, out, M, N, K, s),
                         "mul_mat gemm launch");
}

GroupedKernels q6_K_kernels() {
    // small batch measured at N = 4096..28672: 18.9 against 78 us (GEMV) at
    // M = 8, N = K = 8192; 74 against 77 us (GEMM) at M = 64, N = 28672
    return GroupedKernels{"Q6_K", qmm::q6_K_max_k(), qmm::launch_gemv_q6_K, qmm::launch_gemm_q6_K,
                          qmm::launch_skinny_q6_K, qmm::skinny_q6_K_max_m(), 8 * 8192};
}
GroupedKernels q2_K_kernels() {
    // small batch measured at N = 4096..28672, K = 4096..14336: 11.7 against
    // 32.1 us (GEMV) at M = 8, N = K = 8192; 19.4 against 22.8 us (GEMV at
    // M = 2) at M = 3, N = 28672; 54.6 against 50.4 us (GEMM) at M = 64,
    // N = 28672, 96.6 against 98.9 at M = 256, N = 8192
    return GroupedKernels{"Q2_K", qmm::q2_K_max_k(), qmm::launch_gemv_q2_K, qmm::launch_gemm_q2_K,
                          qmm::launch_skinny_q2_K, qmm::skinny_q2_K_max_m(), 6 * 8192};
}

}  // namespace

extern "C" {

qmm_status qmm_mul_mat_q6_K_ex(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                               size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                               int64_t K, qmm_algo algo, void *stream) {
    return mul_mat_grouped(QMM_Q6_K, q6_K_kernels(), w, w_bytes, l, y, y_bytes, out, out_bytes, M, N,
                           K, algo, stream);
}

qmm_status qmm_mul_mat_q6_K(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                            size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                            int64_t K, void *stream) {
    return qmm_mul_mat_q6_K_ex(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, QMM_ALGO_AUTO,
                               stream);
}

qmm_status qmm_mul_mat_q2_K_ex(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                               size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                               int64_t K, qmm_algo algo, void *stream) {
    return mul_mat_grouped(QMM_Q2_K, q2_K_kernels(), w, w_bytes, l, y, y_bytes, out, out_bytes, M, N,
                           K, algo, stream);
}

qmm_status qmm_mul_mat_q2_K(const void *w, size_t w_bytes, qmm_layout l, const void *y,
                            size_t y_bytes, float *out, size_t out_bytes, int64_t M, int64_t N,
                            int64_t K, void *stream) {
    return qmm_mul_mat_q2_K_ex(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, QMM_ALGO_AUTO,
                               stream);
}


}  // extern "C"

namespace {

// The kernels each weight format uses for mul_mat_id.
struct IdKernels {
    int64_t gemv_max_k;
    bool gemm_canonical;  // the GEMM also reads the canonical layout
    int64_t gemm_k_mult;  // the GEMM's K step
    hipError_t (*gemv)(const uint8_t *, bool, int64_t, const uint8_t *, int, const int32_t *, int64_t, int64_t,
                       int64_t, float *, int64_t, int64_t, hipStream_t);
    hipError_t (*gemm)(const uint8_t *, bool, int64_t, const uint8_t *, int64_t, int, int64_t, const int32_t *,
                       int64_t, int64_t, float *, int64_t, int64_t, hipStream_t);
};

template <hipError_t (*G)(const uint8_t *, int64_t, const uint8_t *, int64_t, int, int64_t, const int32_t *,
                          int64_t, int64_t, float *, int64_t, int64_t, hipStream_t)>
hipError_t gemm_id_repacked(const uint8_t *w, bool, int64_t w_stride, const uint8_t *y, int64_t y_rows,
                            int y_per_slot, int64_t U, const int32_t *ws, int64_t E, int64_t P, float *out,
                            int64_t N, int64_t K, hipStream_t s) {
    return G(w, w_stride, y, y_rows, y_per_slot, U, ws, E, P, out, N, K, s);
}

bool id_kernels(qmm_weight_type t, IdKernels &k) {
    switch (t) {
        case QMM_Q4_K:
            k = IdKernels{qmm::gemv1_max_k(), true, 256, qmm::launch_gemv_id_q4_K, qmm::launch_gemm_id_q4_K};
            return true;
        case QMM_Q6_K:
            k = IdKernels{qmm::q6_K_max_k(), false, 256, qmm::launch_gemv_id_q6_K,
                          gemm_id_repacked<qmm::launch_gemm_id_q6_K>};
            return true;
        case QMM_Q2_K:
            k = IdKernels{qmm::q2_K_max_k(), false, 256, qmm::launch_gemv_id_q2_K,
                          gemm_id_repacked<qmm::launch_gemm_id_q2_K>};
            return true;
        case QMM_Q4_0:  // the GEMV reads whole Q8_0 rows from global memory: no K limit of its own
            k = IdKernels{kMaxK, false, 256, qmm::launch_gemv_id_q4_0,
                          gemm_id_repacked<qmm::launch_gemm_id_q4_0>};
            return true;
    }
    return false;
}

}  // namespace

extern "C" {

size_t qmm_mul_mat_id_workspace_bytes(int64_t T, int64_t U, int64_t E) {
    if (T < 0 || U < 1 || E < 1 || E > qmm::kMoeMaxExperts || T * U > (int64_t(1) << 31) - 1) return 0;
    return (size_t)qmm::moe_group_layout(T * U, E, qmm::gemm_tile_rows()).words * 4;
}

}  // extern "C"

namespace {

// mul_mat_id with the grouping tables in the caller's workspace
// (own_scratch = false) or in the library's per-GPU scratch array.
qmm_status mul_mat_id_impl(qmm_weight_type t, const void *w, size_t w_bytes, int64_t E, qmm_layout l,
                           const void *y, size_t y_bytes, int y_per_slot, const int32_t *ids, int64_t T,
                           int64_t U, float *out, size_t out_bytes, int64_t N, int64_t K, void *workspace,
                           size_t ws_bytes, bool own_scratch, qmm_algo algo, void *stream) {
    IdKernels kk;
    if (!id_kernels(t, kk)) return fail(QMM_EUNSUPPORTED, "unknown weight type %d", (int)t);
    if (algo != QMM_ALGO_AUTO && algo != QMM_ALGO_GEMV && algo != QMM_ALGO_MFMA)
        return fail(QMM_EUNSUPPORTED, "mul_mat_id takes the GEMV or MFMA path (algo %d)", (int)algo);
    if (l != QMM_LAYOUT_CANONICAL && l != QMM_LAYOUT_REPACKED)
        return fail(QMM_EUNSUPPORTED, "unknown layout %d", (int)l);
    if (E < 1 || E > qmm::kMoeMaxExperts)
        return fail(QMM_EUNSUPPORTED, "E = %lld experts; 1 <= E <= %d", (long long)E, qmm::kMoeMaxExperts);
    if (U < 1 || U > E) return fail(QMM_EINVAL, "U = %lld slots per token; 1 <= U <= E", (long long)U);
    if (y_per_slot != 0 && y_per_slot != 1) return fail(QMM_EINVAL, "y_per_slot must be 0 or 1");
    QMM_TRY(check_rows("T", T));
    QMM_TRY(check_rows("N", N));
    QMM_TRY(check_k(K, w_qk(t)));
    const int64_t P = T * U;
    if (P > (int64_t(1) << 31) - 1) return fail(QMM_EUNSUPPORTED, "T*U = %lld pairs exceeds 2^31 - 1", (long long)P);
    if (P == 0 || N == 0) return QMM_OK;
    const qmm_act_type at = t == QMM_Q4_0 ? QMM_Q8_0 : QMM_Q8_K;
    const int64_t y_rows = y_per_slot ? P : T;
    const size_t w_one = qmm_weight_bytes(t, l, N, K);
    QMM_TRY(check_ptr("w", w));
    QMM_TRY(check_ptr("y", y));
    QMM_TRY(check_ptr("ids", ids));
    QMM_TRY(check_ptr("out", out));
    QMM_TRY(check_size("w", w_bytes, w_one * (size_t)E));
    QMM_TRY(check_size("y", y_bytes, qmm_act_bytes(at, y_rows, K)));
    QMM_TRY(check_size("out", out_bytes, (size_t)(P * N) * sizeof(float)));
    const bool gemv_ok = K <= kk.gemv_max_k;
    // the grouped GEMMs address one expert matrix and the activations with 32-bit offsets
    const bool mfma_ok = (kk.gemm_canonical || l == QMM_LAYOUT_REPACKED) && K % kk.gemm_k_mult == 0 &&
                         w_one < (size_t(1) << 32) && qmm_act_bytes(at, y_rows, K) < (size_t(1) << 32);
    if (algo == QMM_ALGO_GEMV && !gemv_ok)
        return fail(QMM_EUNSUPPORTED, "mul_mat_id GEMV takes K <= %lld", (long long)kk.gemv_max_k);
    if (algo == QMM_ALGO_MFMA && !mfma_ok)
        return fail(QMM_EUNSUPPORTED,
                    "mul_mat_id MFMA path: this format needs the repacked layout, K a multiple of %lld and "
                    "matrices below 4 GiB", (long long)kk.gemm_k_mult);
    if (algo == QMM_ALGO_AUTO && !gemv_ok && !mfma_ok)
        return fail(QMM_EUNSUPPORTED, "no mul_mat_id kernel takes this call (K = %lld)", (long long)K);
    qmm_algo a = algo;
    // AUTO: a per-pair GEMV streams one expert matrix per pair; the grouped
    // GEMM reads each routed expert once but at a lower rate when its tiles are
    // sparse.  Measured on eight 14336 x 4096 Q4_K experts the two cross between
    // 32 and 48 pairs, i.e. near four pairs per expert.
    if (a == QMM_ALGO_AUTO) a = (P <= 4 * E && gemv_ok) || !mfma_ok ? QMM_ALGO_GEMV : QMM_ALGO_MFMA;
    if (log_enabled())
        fprintf(stderr, "qmm: mul_mat_id %s E=%lld T=%lld U=%lld N=%lld K=%lld layout=%s algo=%s -> %s (%s)\n",
                t == QMM_Q4_0 ? "Q4_0" : t == QMM_Q4_K ? "Q4_K" : t == QMM_Q6_K ? "Q6_K" : "Q2_K", (long long)E,
                (long long)T, (long long)U, (long long)N, (long long)K,
                l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical", algo_name(algo), algo_name(a),
                a == QMM_ALGO_GEMV ? "one M = 1 GEMV per (token, slot)"
                                   : "expert grouping, then 128 x 256 tiles of each expert's rows");
    hipStream_t s = static_cast<hipStream_t>(stream);
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const uint8_t *yb = static_cast<const uint8_t *>(y);
    const bool rep = l == QMM_LAYOUT_REPACKED;
    if (a == QMM_ALGO_GEMV)
        return device_status(kk.gemv(wb, rep, (int64_t)w_one, yb, y_per_slot, ids, P, U, E, out, N, K, s),
                             "mul_mat_id gemv launch");
    int32_t *ws = nullptr;
    if (own_scratch) {
        QMM_TRY(device_status(qmm::noalloc_scratch(s, &ws), "mul_mat_id scratch address"));
    } else {
        QMM_TRY(check_ptr("workspace", workspace));
        QMM_TRY(check_size("workspace", ws_bytes, qmm_mul_mat_id_workspace_bytes(T, U, E)));
        ws = static_cast<int32_t *>(workspace);
    }
    QMM_TRY(device_status(qmm::launch_moe_group_ids(ids, P, E, ws, out, N, s), "mul_mat_id grouping launch"));
    return device_status(kk.gemm(wb, rep, (int64_t)w_one, yb, y_rows, y_per_slot, U, ws, E, P, out, N, K, s),
                         "mul_mat_id gemm launch");
}

}  // namespace

extern "C" {

qmm_status qmm_mul_mat_id(qmm_weight_type t, const void *w, size_t w_bytes, int64_t E, qmm_layout l,
                          const void *y, size_t y_bytes, int y_per_slot, const int32_t *ids, int64_t T,
                          int64_t U, float *out, size_t out_bytes, int64_t N, int64_t K, void *workspace,
                          size_t ws_bytes, qmm_algo algo, void *stream) {
    return mul_mat_id_impl(t, w, w_bytes, E, l, y, y_bytes, y_per_slot, ids, T, U, out, out_bytes, N, K,
                           workspace, ws_bytes, false, algo, stream);
}

qmm_status qmm_mul_mat_id_noalloc(qmm_weight_type t, const void *w, size_t w_bytes, int64_t E, qmm_layout l,
                                  const void *y, size_t y_bytes, int y_per_slot, const int32_t *ids,
                                  int64_t T, int64_t U, float *out, size_t out_bytes, int64_t N, int64_t K,
                                  qmm_algo algo, void *stream) {
    // the grouping must fit the library's scratch array (checked before any
    // HIP call; only the per-pair GEMV path needs no grouping)
    const size_t need = qmm_mul_mat_id_workspace_bytes(T, U, E);
    if (algo != QMM_ALGO_GEMV && need > qmm::kNoAllocScratchBytes)
        return fail(QMM_EUNSUPPORTED,
                    "mul_mat_id_noalloc: the expert grouping of T = %lld, U = %lld, E = %lld needs %zu bytes; "
                    "the library's scratch holds %zu (use qmm_mul_mat_id with a workspace, or QMM_ALGO_GEMV)",
                    (long long)T, (long long)U, (long long)E, need, qmm::kNoAllocScratchBytes);
    return mul_mat_id_impl(t, w, w_bytes, E, l, y, y_bytes, y_per_slot, ids, T, U, out, out_bytes, N, K,
                           nullptr, 0, true, algo, stream);
}

qmm_status qmm_mul_mat_id_q4_K(const void *w, size_t w_bytes, int64_t E, qmm_layout l, const void *y,
                               size_t y_bytes, int y_per_slot, const int32_t *ids, int64_t T,
                               int64_t U, float *out, size_t out_bytes, int64_t N, int64_t K,
                               void *workspace, size_t ws_bytes, qmm_algo algo, void *stream) {
    return qmm_mul_mat_id(QMM_Q4_K, w, w_bytes, E, l, y, y_bytes, y_per_slot, ids, T, U, out, out_bytes, N, K,
                          workspace, ws_bytes, algo, stream);
}

qmm_status qmm_quantize_mul_mat(qmm_weight_type t, const void *w, size_t w_bytes, qmm_layout l,
                                const float *x, void *y, size_t y_bytes, float *out,
                                size_t out_bytes, int64_t M, int64_t N, int64_t K, void *stream) {
    if (!w_qk(t)) return fail(QMM_EUNSUPPORTED, "unknown weight type %d", (int)t);
    if (l != QMM_LAYOUT_CANONICAL && l != QMM_LAYOUT_REPACKED)
        return fail(QMM_EUNSUPPORTED, "unknown layout %d", (int)l);
    const qmm_act_type at = t == QMM_Q4_0 ? QMM_Q8_0 : QMM_Q8_K;
    QMM_TRY(check_rows("M", M));
    QMM_TRY(check_rows("N", N));
    QMM_TRY(check_k(K, w_qk(t)));
    if (M == 0) return QMM_OK;
    QMM_TRY(check_ptr("x", x));
    QMM_TRY(check_ptr("y", y));
    QMM_TRY(check_size("y", y_bytes, qmm_act_bytes(at, M, K)));
    if (N > 0) {
        QMM_TRY(check_ptr("w", w));
        QMM_TRY(check_ptr("out", out));
        QMM_TRY(check_size("w", w_bytes, qmm_weight_bytes(t, l, N, K)));
        QMM_TRY(check_size("out", out_bytes, (size_t)(M * N) * sizeof(float)));
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    uint8_t *yb = static_cast<uint8_t *>(y);
    if (t == QMM_Q4_K && M == 1 && N > 0 && K <= qmm::gemv1_fused_max_k()) {
        if (log_enabled())
            fprintf(stderr, "qmm: quantize_mul_mat Q4_K M=1 N=%lld K=%lld layout=%s -> fused quantize + GEMV "
                    "(one launch, one wavefront per output row)\n", (long long)N, (long long)K,
                    l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical");
        return device_status(qmm::launch_gemv1_fused_q4_K(static_cast<const uint8_t *>(w),
                                                          l == QMM_LAYOUT_REPACKED, x, yb, out, N,
                                                          K, s),
                             "quantize_mul_mat fused launch");
    }
    if (t == QMM_Q6_K && M == 1 && N > 0 && qmm::gemv_fused_q6_K_ok(N, K)) {
        if (log_enabled())
            fprintf(stderr, "qmm: quantize_mul_mat Q6_K M=1 N=%lld K=%lld layout=%s -> fused quantize + GEMV "
                    "(one launch, one wavefront per output row)\n", (long long)N, (long long)K,
                    l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical");
        return device_status(qmm::launch_gemv_fused_q6_K(static_cast<const uint8_t *>(w),
                                                         l == QMM_LAYOUT_REPACKED, x, yb, out, N, K, s),
                             "quantize_mul_mat fused launch");
    }
    if (t == QMM_Q2_K && M == 1 && N > 0 && qmm::gemv_fused_q2_K_ok(N, K)) {
        if (log_enabled())
            fprintf(stderr, "qmm: quantize_mul_mat Q2_K M=1 N=%lld K=%lld layout=%s -> fused quantize + GEMV "
                    "(one launch, one wavefront per output row)\n", (long long)N, (long long)K,
                    l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical");
        return device_status(qmm::launch_gemv_fused_q2_K(static_cast<const uint8_t *>(w),
                                                         l == QMM_LAYOUT_REPACKED, x, yb, out, N, K, s),
                             "quantize_mul_mat fused launch");
    }
    if (t == QMM_Q4_0 && M == 1 && N > 0 && qmm::gemv_fused_q4_0_ok(N, K)) {
        if (log_enabled())
            fprintf(stderr, "qmm: quantize_mul_mat Q4_0 M=1 N=%lld K=%lld layout=%s -> fused quantize + GEMV "
                    "(one launch, one wavefront per output row)\n", (long long)N, (long long)K,
                    l == QMM_LAYOUT_REPACKED ? "repacked" : "canonical");
        return device_status(qmm::launch_gemv_fused_q4_0(static_cast<const uint8_t *>(w),
                                                         l == QMM_LAYOUT_REPACKED, x, yb, out, N, K, s),
                             "quantize_mul_mat fused launch");
    }
    QMM_TRY(qmm_quantize_row_q8(at, x, M, K, y, y_bytes, stream));
    if (N == 0) return QMM_OK;
    if (t == QMM_Q6_K) return qmm_mul_mat_q6_K(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, stream);
    if (t == QMM_Q2_K) return qmm_mul_mat_q2_K(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, stream);
    return t == QMM_Q4_K ? qmm_mul_mat_q4_K(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, stream)
                         : qmm_mul_mat_q4_0(w, w_bytes, l, y, y_bytes, out, out_bytes, M, N, K, stream);
}

qmm_status qmm_debug_block_sums(qmm_weight_type t, const void *w, size_t w_bytes, qmm_layout l,
                                const void *y, size_t y_bytes, int32_t *P, size_t p_bytes,
                                int64_t M, int64_t N, int64_t K, void *stream) {
    if (!w_qk(t)) return fail(QMM_EUNSUPPORTED, "unknown weight type %d", (int)t);
    QMM_TRY(mul_mat_common(t, w, w_bytes, l, y, y_bytes, reinterpret_cast<const float *>(P),
                           p_bytes, M, N, K));
    if ((t == QMM_Q6_K || t == QMM_Q2_K) && K > qmm::q8k_group_max_k())
        return fail(QMM_EUNSUPPORTED, "group sums take K <= %lld (K = %lld)",
                    (long long)qmm::q8k_group_max_k(), (long long)K);
    if (M == 0 || N == 0) return QMM_OK;
    const int64_t group = (t == QMM_Q6_K || t == QMM_Q2_K) ? 16 : 32;
    QMM_TRY(check_size("P", p_bytes, (size_t)(M * N * (K / group)) * sizeof(int32_t)));
    hipStream_t s = static_cast<hipStream_t>(stream);
    const bool rep = l == QMM_LAYOUT_REPACKED;
    const uint8_t *wb = static_cast<const uint8_t *>(w);
    const uint8_t *yb = static_cast<const uint8_t *>(y);
    return device_status(t == QMM_Q4_K   ? qmm::launch_block_sums_q4_K(wb, rep, yb, P, M, N, K, s)
                         : t == QMM_Q6_K ? qmm::launch_group_sums_q6_K(wb, rep, yb, P, M, N, K, s)
                         : t == QMM_Q2_K ? qmm::launch_group_sums_q2_K(wb, rep, yb, P, M, N, K, s)
                                         : qmm::launch_block_sums_q4_0(wb, rep, yb, P, M, N, K, s),
                         "debug_block_sums launch");
}

const char *qmm_status_string(qmm_status s) {
    switch (s) {
        case QMM_OK: return "ok";
        case QMM_EINVAL: return "invalid argument";
        case QMM_EALIGN: return "pointer not 16-byte aligned";
        case QMM_EUNSUPPORTED: return "unsupported shape or option";
        case QMM_EDEVICE: return "HIP runtime error";
    }
    return "unknown status";
}

const char *qmm_last_error(void) { return g_err; }

const char *qmm_version(void) { return "qmm 0.1.0 (gfx950)"; }

}  // extern "C"
