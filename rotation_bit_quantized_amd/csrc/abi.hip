// The exported C ABI (include/qr.h): argument validation on the host, then
// dispatch to the kernels.  Nothing here allocates or synchronises; the only
// state kept is, per device, the address of the static scratch array below
// (and the CU count, in the launchers); a rejected call launches nothing.
#include "../../include/qr.h"
#include "qr_launch.h"

#include <atomic>
#include <mutex>

// Scratch memory of qr_kv_attn_decode_noalloc (the split partials of decode
// attention): one copy per GPU, part of the library's code object, held until
// the process ends.  In host code `scratch` names a host-side stand-in, not a
// device address: the device address is taken with hipGetSymbolAddress, once
// per device, and only that pointer is ever handed to a kernel.
constexpr int64_t kScratchBytes = (int64_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];            // written once per device under g_scratch_mu
std::atomic<bool> g_scratch_ready[kMaxDevices];

// The device address of `scratch` on the current device (looked up on the
// first call on that device, with that device current).
qr_status scratch_on_current_device(void **ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QR_EDEVICE;
  if (!g_scratch_ready[dev].load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ready[dev].load(std::memory_order_relaxed)) {
      void *p = nullptr;
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return QR_EDEVICE;
      g_scratch_ptr[dev] = p;
      g_scratch_ready[dev].store(true, std::memory_order_release);
    }
  }
  *ptr = g_scratch_ptr[dev];
  return QR_OK;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }
inline bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

qr_status from_hip(hipError_t e) { return e == hipSuccess ? QR_OK : QR_EDEVICE; }

qr_status check_rotation(const qr_rotation *rot) {
  if (rot == nullptr) return QR_EINVAL;
  if (rot->n <= 0 || rot->had_n <= 0 || rot->dense_m <= 0) return QR_EINVAL;
  if (!pow2(rot->had_n) || rot->had_n > 32768) return QR_ESHAPE;
  if (rot->dense_m > 256) return QR_ESHAPE;
  if (rot->n != rot->had_n * rot->dense_m) return QR_ESHAPE;
  if (rot->n < 2 || rot->n > 32768 || (rot->n & 1)) return QR_ESHAPE;
  // rows wider than 16384 are transformed in place in LDS: small dense factors only
  if (rot->n > 16384 && rot->dense_m > 16) return QR_ESHAPE;
  if ((rot->dense == nullptr) != (rot->dense_m == 1)) return QR_EINVAL;
  if (rot->dense != nullptr && !aligned(rot->dense, 4)) return QR_EALIGN;
  return QR_OK;
}

qr_status check_gemm(const uint8_t *a, const uint8_t *w, int64_t M, int64_t N, int64_t K, int64_t group) {
  if (M < 0 || N < 0 || K <= 0) return QR_EINVAL;
  // |product| <= 128 * 128 = 2^14 (8-bit codes, or 4-bit codes widened to
  // 16 q): int32 sums stay exact while K * 2^14 < 2^31, i.e. K < 2^17
  // (largest valid K: 130944)
  if (K % 128 != 0 || K >= (int64_t)1 << 17) return QR_ESHAPE;
  if (group != 0 && (group < 128 || group % 128 != 0 || K % group != 0)) return QR_ESHAPE;
  if (M > ((int64_t)1 << 30) || N > ((int64_t)1 << 30)) return QR_ESHAPE;
  if (M == 0 || N == 0) return QR_OK;
  if (a == nullptr || w == nullptr) return QR_EINVAL;
  if (!aligned(a, 16) || !aligned(w, 16)) return QR_EALIGN;
  return QR_OK;
}

qr_status check_attn(const void *q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t head_dim,
                     const uint8_t *k_codes, const float *k_scales, const uint8_t *k_zeros, const uint8_t *v_codes,
                     const float *v_scales, const uint8_t *v_zeros, const int32_t *lens, const int8_t *signs,
                     float sm_scale, const void *out_f16) {
  if (B < 0 || Hq < 0 || Hkv < 0 || T < 0) return QR_EINVAL;
  if (head_dim != 128) return QR_ESHAPE;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return QR_ESHAPE;
  if (B > 65535 || Hq > 65535 || T > ((int64_t)1 << 30) || B * T * Hkv > ((int64_t)1 << 40)) return QR_ESHAPE;
  if (T * Hkv * 64 >= ((int64_t)1 << 31)) return QR_ESHAPE;   // one sequence's cache rows: 32-bit byte offsets
  if (!(sm_scale == sm_scale) || sm_scale > 3.0e38f || sm_scale < -3.0e38f) return QR_EINVAL;
  if (B == 0 || Hq == 0) return QR_OK;
  if (q_f16 == nullptr || out_f16 == nullptr) return QR_EINVAL;
  if (T > 0 && (k_codes == nullptr || k_scales == nullptr || k_zeros == nullptr || v_codes == nullptr ||
                v_scales == nullptr || v_zeros == nullptr))
    return QR_EINVAL;
  if (!aligned(q_f16, 2) || !aligned(out_f16, 2)) return QR_EALIGN;
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(k_scales, 4) || !aligned(v_scales, 4))
    return QR_EALIGN;
  if ((lens != nullptr && !aligned(lens, 4)) || (signs != nullptr && !aligned(signs, 4))) return QR_EALIGN;
  return QR_OK;
}

}  // namespace

extern "C" {

const char *qr_status_str(qr_status s) {
  switch (s) {
    case QR_OK: return "ok";
    case QR_EINVAL: return "invalid argument (null pointer, negative size or bad value)";
    case QR_ESHAPE: return "unsupported shape";
    case QR_EALIGN: return "misaligned pointer or leading dimension";
    case QR_EDEVICE: return "HIP runtime error at launch";
    case QR_ESCRATCH: return "the call needs more scratch memory than the library's static buffer holds";
  }
  return "unknown status";
}

int qr_version(void) { return 100; }

qr_status qr_rotate_quant(const void *x_f16, int64_t rows, int64_t ld_x, const qr_rotation *rot,
                          int64_t group, uint8_t *codes, float *scales, void *stream) {
  qr_status st = check_rotation(rot);
  if (st != QR_OK) return st;
  if (rows < 0) return QR_EINVAL;
  if (group != 0 && (group < 32 || !pow2(group) || rot->n % group != 0)) return QR_ESHAPE;
  if (ld_x < rot->n) return QR_ESHAPE;
  if (ld_x % 8 != 0) return QR_EALIGN;
  if (rows == 0) return QR_OK;
  if (x_f16 == nullptr || codes == nullptr || scales == nullptr) return QR_EINVAL;
  if (!aligned(x_f16, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return QR_EALIGN;
  if (rot->signs != nullptr && !aligned(rot->signs, 4)) return QR_EALIGN;

  qr::RotArgs r{(int)rot->n, (int)rot->had_n, (int)rot->dense_m, rot->dense, rot->signs};
  hipStream_t s = (hipStream_t)stream;
  if (qr::rq_pow2_supported(r, (int)group))
    return from_hip(qr::launch_rq_pow2(x_f16, rows, ld_x, r, (int)group, codes, scales, s));
  if (qr::rq_kron_supported(r, (int)group))
    return from_hip(qr::launch_rq_kron(x_f16, rows, ld_x, r, (int)group, codes, scales, s));
  if (qr::rq_kron4096_supported(r, (int)group))
    return from_hip(qr::launch_rq_kron4096(x_f16, rows, ld_x, r, codes, scales, s));
  return from_hip(qr::launch_rq_generic(x_f16, rows, ld_x, r, (int)group, codes, scales, s));
}

qr_status qr_rotate_quant_i8(const void *x_f16, int64_t rows, int64_t ld_x, const qr_rotation *rot,
                             int64_t group, int64_t bits, int8_t *codes, float *scales, void *stream) {
  qr_status st = check_rotation(rot);
  if (st != QR_OK) return st;
  if (bits != 6 && bits != 8) return QR_EINVAL;
  if (rows < 0) return QR_EINVAL;
  if (group != 0 && (group < 32 || !pow2(group) || rot->n % group != 0)) return QR_ESHAPE;
  if (ld_x < rot->n) return QR_ESHAPE;
  if (ld_x % 8 != 0) return QR_EALIGN;
  if (rows == 0) return QR_OK;
  if (x_f16 == nullptr || codes == nullptr || scales == nullptr) return QR_EINVAL;
  if (!aligned(x_f16, 16) || !aligned(codes, 16) || !aligned(scales, 4)) return QR_EALIGN;
  if (rot->signs != nullptr && !aligned(rot->signs, 4)) return QR_EALIGN;

  qr::RotArgs r{(int)rot->n, (int)rot->had_n, (int)rot->dense_m, rot->dense, rot->signs};
  hipStream_t s = (hipStream_t)stream;
  if (qr::rq_pow2_supported(r, (int)group))
    return from_hip(qr::launch_rq_pow2_bits(x_f16, rows, ld_x, r, (int)group, (int)bits, (uint8_t *)codes, scales, s));
  return from_hip(
      qr::launch_rq_generic_bits(x_f16, rows, ld_x, r, (int)group, (int)bits, (uint8_t *)codes, scales, s));
}

qr_status qr_swiglu_rotate_quant(const void *gate_f16, const void *up_f16, int64_t rows, int64_t ld,
                                 const qr_rotation *rot, int64_t group, uint8_t *codes, float *scales,
                                 void *stream) {
  qr_status st = check_rotation(rot);
  if (st != QR_OK) return st;
  if (rows < 0) return QR_EINVAL;
  if (group != 0 && (group < 32 || !pow2(group) || rot->n % group != 0)) return QR_ESHAPE;
  if (ld < rot->n) return QR_ESHAPE;
  if (ld % 8 != 0) return QR_EALIGN;
  if (rows == 0) return QR_OK;
  if (gate_f16 == nullptr || up_f16 == nullptr || codes == nullptr || scales == nullptr) return QR_EINVAL;
  if (!aligned(gate_f16, 16) || !aligned(up_f16, 16) || !aligned(codes, 16) || !aligned(scales, 4))
    return QR_EALIGN;
  if (rot->signs != nullptr && !aligned(rot->signs, 4)) return QR_EALIGN;

  qr::RotArgs r{(int)rot->n, (int)rot->had_n, (int)rot->dense_m, rot->dense, rot->signs};
  hipStream_t s = (hipStream_t)stream;
  if (qr::rq_kron4096_supported(r, (int)group))
    return from_hip(qr::launch_swiglu_rq_kron4096(gate_f16, up_f16, rows, ld, r, codes, scales, s));
  return from_hip(qr::launch_rq_generic_full(gate_f16, up_f16, rows, ld, r, (int)group, 4, codes, scales, s));
}

qr_status qr_int8_gemm(const int8_t *a_codes, const float *a_scales, const int8_t *w_codes,
                       const float *w_scales, int64_t M, int64_t N, int64_t K, int64_t group, void *y_f16,
                       int64_t ld_y, void *stream) {
  qr_status st = check_gemm((const uint8_t *)a_codes, (const uint8_t *)w_codes, M, N, K, group);
  if (st != QR_OK) return st;
  if (ld_y < N) return QR_ESHAPE;
  if (M == 0 || N == 0) return QR_OK;
  if (a_scales == nullptr || w_scales == nullptr || y_f16 == nullptr) return QR_EINVAL;
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(y_f16, 2)) return QR_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M <= 64)
    return from_hip(qr::launch_gemm_decode_i8(a_codes, a_scales, w_codes, w_scales, M, N, K, (int)group, y_f16,
                                              ld_y, false, s));
  return from_hip(qr::launch_gemm_prefill_i8(a_codes, a_scales, w_codes, w_scales, M, N, K, (int)group, y_f16,
                                             ld_y, false, s));
}

qr_status qr_int8_gemm_i32(const int8_t *a_codes, const int8_t *w_codes, int64_t M, int64_t N, int64_t K,
                           int64_t group, int32_t *acc, void *stream) {
  qr_status st = check_gemm((const uint8_t *)a_codes, (const uint8_t *)w_codes, M, N, K, group);
  if (st != QR_OK) return st;
  if (M == 0 || N == 0) return QR_OK;
  if (acc == nullptr) return QR_EINVAL;
  if (!aligned(acc, 4)) return QR_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M <= 64)
    return from_hip(qr::launch_gemm_decode_i8(a_codes, nullptr, w_codes, nullptr, M, N, K, (int)group, acc, N,
                                              true, s));
  return from_hip(qr::launch_gemm_prefill_i8(a_codes, nullptr, w_codes, nullptr, M, N, K, (int)group, acc, N,
                                             true, s));
}

qr_status qr_int4_gemm(const uint8_t *a_codes, const float *a_scales, const uint8_t *w_codes,
                       const float *w_scales, int64_t M, int64_t N, int64_t K, int64_t group, void *y_f16,
                       int64_t ld_y, void *stream) {
  qr_status st = check_gemm(a_codes, w_codes, M, N, K, group);
  if (st != QR_OK) return st;
  if (ld_y < N) return QR_ESHAPE;
  if (M == 0 || N == 0) return QR_OK;
  if (a_scales == nullptr || w_scales == nullptr || y_f16 == nullptr) return QR_EINVAL;
  if (!aligned(a_scales, 4) || !aligned(w_scales, 4) || !aligned(y_f16, 2)) return QR_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M <= 64)
    return from_hip(qr::launch_gemm_decode(a_codes, a_scales, w_codes, w_scales, M, N, K, (int)group, y_f16,
                                           ld_y, false, s));
  return from_hip(qr::launch_gemm_prefill(a_codes, a_scales, w_codes, w_scales, M, N, K, (int)group, y_f16,
                                          ld_y, false, s));
}

qr_status qr_int4_gemm_i32(const uint8_t *a_codes, const uint8_t *w_codes, int64_t M, int64_t N, int64_t K,
                           int64_t group, int32_t *acc, void *stream) {
  qr_status st = check_gemm(a_codes, w_codes, M, N, K, group);
  if (st != QR_OK) return st;
  if (M == 0 || N == 0) return QR_OK;
  if (acc == nullptr) return QR_EINVAL;
  if (!aligned(acc, 4)) return QR_EALIGN;
  hipStream_t s = (hipStream_t)stream;
  if (M <= 64)
    return from_hip(qr::launch_gemm_decode(a_codes, nullptr, w_codes, nullptr, M, N, K, (int)group, acc, N,
                                           true, s));
  return from_hip(qr::launch_gemm_prefill(a_codes, nullptr, w_codes, nullptr, M, N, K, (int)group, acc, N,
                                          true, s));
}

qr_status qr_kv_quant(const void *kv_f16, int64_t T, int64_t H, int64_t head_dim, int64_t ld_kv,
                      const int8_t *signs, uint8_t *codes, float *scales, uint8_t *zeros, void *stream) {
  if (T < 0 || H < 0) return QR_EINVAL;
  if (head_dim != 128) return QR_ESHAPE;
  if (H > ((int64_t)1 << 20)) return QR_ESHAPE;
  if (ld_kv < H * head_dim) return QR_ESHAPE;
  if (ld_kv % 8 != 0) return QR_EALIGN;
  if (T == 0 || H == 0) return QR_OK;
  if (kv_f16 == nullptr || codes == nullptr || scales == nullptr || zeros == nullptr) return QR_EINVAL;
  if (!aligned(kv_f16, 16) || !aligned(codes, 4) || !aligned(scales, 4)) return QR_EALIGN;
  if (signs != nullptr && !aligned(signs, 4)) return QR_EALIGN;
  return from_hip(qr::launch_kv_quant(kv_f16, T, H, ld_kv, signs, codes, scales, zeros, (hipStream_t)stream));
}

qr_status qr_kv_attn_decode_workspace(int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t head_dim,
                                      int64_t *bytes) {
  if (bytes == nullptr || B < 0 || Hq < 0 || Hkv < 0 || T < 0) return QR_EINVAL;
  if (head_dim != 128) return QR_ESHAPE;
  if (Hq > 0 && (Hkv == 0 || Hq % Hkv != 0)) return QR_ESHAPE;
  *bytes = qr::attn_decode_plan(B, Hq, Hkv, T).workspace_bytes;
  return QR_OK;
}

qr_status qr_kv_attn_decode(const void *q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t T, int64_t head_dim,
                            const uint8_t *k_codes, const float *k_scales, const uint8_t *k_zeros,
                            const uint8_t *v_codes, const float *v_scales, const uint8_t *v_zeros,
                            const int32_t *lens, const int8_t *signs, float sm_scale, void *workspace,
                            int64_t workspace_bytes, void *out_f16, void *stream) {
  qr_status st = check_attn(q_f16, B, Hq, Hkv, T, head_dim, k_codes, k_scales, k_zeros, v_codes, v_scales,
                            v_zeros, lens, signs, sm_scale, out_f16);
  if (st != QR_OK) return st;
  if (workspace_bytes < 0) return QR_EINVAL;
  if (B == 0 || Hq == 0) return QR_OK;
  qr::AttnPlan plan = qr::attn_decode_plan(B, Hq, Hkv, T);
  if (plan.splits > 1) {
    if (workspace == nullptr && workspace_bytes == 0) {
      // no workspace: one chunk per sequence
      plan.chunk = (T + 15) / 16 * 16;
      plan.splits = 1;
      plan.tiles = plan.gqa ? B * Hkv : B * plan.nhg;
      plan.blocks = plan.gqa ? plan.tiles : (plan.tiles + 7) / 8 * 8 * (Hq / Hkv);
      plan.workspace_bytes = 0;
    } else if (workspace == nullptr || workspace_bytes < plan.workspace_bytes) {
      return QR_EINVAL;
    } else if (!aligned(workspace, 16)) {
      return QR_EALIGN;
    }
  }
  return from_hip(qr::launch_attn_decode(q_f16, B, Hq, Hkv, T, k_codes, k_scales, k_zeros, v_codes, v_scales,
                                         v_zeros, lens, signs, sm_scale, plan, (float *)workspace, out_f16,
                                         (hipStream_t)stream));
}

qr_status qr_kv_attn_decode_noalloc(const void *q_f16, int64_t B, int64_t Hq, int64_t Hkv, int64_t T,
                                    int64_t head_dim, const uint8_t *k_codes, const float *k_scales,
                                    const uint8_t *k_zeros, const uint8_t *v_codes, const float *v_scales,
                                    const uint8_t *v_zeros, const int32_t *lens, const int8_t *signs,
                                    float sm_scale, void *out_f16, void *stream) {
  qr_status st = check_attn(q_f16, B, Hq, Hkv, T, head_dim, k_codes, k_scales, k_zeros, v_codes, v_scales,
                            v_zeros, lens, signs, sm_scale, out_f16);
  if (st != QR_OK) return st;
  if (B == 0 || Hq == 0) return QR_OK;
  // the same plan (and so the same kernels and results) as qr_kv_attn_decode
  // with a workspace; the split partials go to the static scratch array
  const qr::AttnPlan plan = qr::attn_decode_plan(B, Hq, Hkv, T);
  if (plan.workspace_bytes > kScratchBytes) return QR_ESCRATCH;
  void *ws = nullptr;
  if (plan.splits > 1) {
    st = scratch_on_current_device(&ws);
    if (st != QR_OK) return st;
  }
  // every partial a launch merges is written by the same launch first: the
  // scratch needs no clearing between calls
  return from_hip(qr::launch_attn_decode(q_f16, B, Hq, Hkv, T, k_codes, k_scales, k_zeros, v_codes, v_scales,
                                         v_zeros, lens, signs, sm_scale, plan, (float *)ws, out_f16,
                                         (hipStream_t)stream));
}

}  // extern "C"
