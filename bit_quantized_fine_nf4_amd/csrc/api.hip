// C ABI: argument validation, workspace sizing and dispatch to the kernels.
// Every check happens before anything is enqueued, so a rejected call leaves
// all outputs untouched.

#include "../../include/qlora_nf4.h"
#include "codec.h"
#include "glue.h"
#include "linear.h"
#include "optim.h"
#include "stream.h"

#include <cmath>
#include <cstddef>

using namespace ql;

namespace {

inline bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline qlora_status_t launch_status(hipError_t e) { return e == hipSuccess ? QLORA_OK : QLORA_ERR_LAUNCH; }

inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// The weight descriptor keeps the layout callers compile against.
static_assert(sizeof(qlora_nf4_weight_t) == 48, "qlora_nf4_weight_t layout");
static_assert(offsetof(qlora_nf4_weight_t, h) == 32 && offsetof(qlora_nf4_weight_t, o) == 40,
              "qlora_nf4_weight_t layout");

bool valid_weight(const qlora_nf4_weight_t *W, int codebook) {
  if (!W || !W->codes || !W->qabsmax || !W->scale2 || !W->mean) return false;
  if (W->h <= 0 || W->o <= 0 || W->h % 64 || W->o % 64) return false;
  if (W->h > (int64_t(1) << 20) || W->o > (int64_t(1) << 20)) return false;
  if (W->h * W->o / 64 >= (int64_t(1) << 32)) return false;
  if (codebook < 0 || codebook >= kCodebooks) return false;
  return aligned(W->codes, 16) && aligned(W->qabsmax, 4) && aligned(W->scale2, 4) && aligned(W->mean, 4);
}

}  // namespace

extern "C" {

const char *qlora_status_string(qlora_status_t s) {
  switch (s) {
    case QLORA_OK: return "success";
    case QLORA_ERR_INVALID_VALUE: return "invalid argument (pointer, size, alignment, rank or workspace)";
    case QLORA_ERR_UNSUPPORTED: return "unsupported request";
    case QLORA_ERR_LAUNCH: return "kernel launch failed";
    case QLORA_ERR_INTERNAL: return "NF4 tables could not be built";
  }
  return "unknown status";
}

qlora_status_t qlora_nf4_levels(float out[16]) {
  if (!out) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables();
  if (!t) return QLORA_ERR_INTERNAL;
  for (int i = 0; i < 16; ++i) out[i] = t->level[i];
  return QLORA_OK;
}

qlora_status_t qlora_merge_adapter_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *L1,
                                      const uint16_t *L2, int32_t r, float s, void *out, qlora_dtype_t out_dtype,
                                      void *stream) {
  if (!valid_weight(W, codebook) || !out || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_INVALID_VALUE;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!L1 || !L2 || !aligned(L1, 16) || !aligned(L2, 16))) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(out, 16)) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  const MergeArgs m{W->codes, W->qabsmax, W->scale2, W->mean, W->h, W->o, L1, L2, r, s, out, nullptr, nullptr};
  return launch_status(launch_merge(m, out_dtype == QLORA_BF16 ? 1 : 0, *t, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_merge_adapter(const qlora_nf4_weight_t *W, const uint16_t *L1, const uint16_t *L2, int32_t r,
                                   float s, void *out, qlora_dtype_t out_dtype, void *stream) {
  return qlora_merge_adapter_cb(W, QLORA_CB_NF4, L1, L2, r, s, out, out_dtype, stream);
}

qlora_status_t qlora_merge_requantize_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *L1,
                                         const uint16_t *L2, int32_t r, float s, uint8_t *codes_out,
                                         float *absmax_out, void *stream) {
  if (!valid_weight(W, codebook) || !codes_out || !absmax_out || r < 0 || r > QLORA_MAX_RANK)
    return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!L1 || !L2 || !aligned(L1, 16) || !aligned(L2, 16))) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(codes_out, 8) || !aligned(absmax_out, 4)) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  const MergeArgs m{W->codes, W->qabsmax, W->scale2, W->mean, W->h, W->o, L1, L2, r, s, nullptr, codes_out,
                    absmax_out};
  return launch_status(launch_merge(m, 2, *t, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_merge_requantize(const qlora_nf4_weight_t *W, const uint16_t *L1, const uint16_t *L2,
                                      int32_t r, float s, uint8_t *codes_out, float *absmax_out, void *stream) {
  return qlora_merge_requantize_cb(W, QLORA_CB_NF4, L1, L2, r, s, codes_out, absmax_out, stream);
}

qlora_status_t qlora_adamw_step(float *param, const float *grad, float *exp_avg, float *exp_avg_sq, int64_t n,
                                int64_t step, float lr, float beta1, float beta2, float eps, float weight_decay,
                                uint16_t *param_bf16, void *stream) {
  if (n < 1 || step < 1 || !param || !grad || !exp_avg || !exp_avg_sq) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(param, 16) || !aligned(grad, 16) || !aligned(exp_avg, 16) || !aligned(exp_avg_sq, 16))
    return QLORA_ERR_INVALID_VALUE;
  if (param_bf16 && !aligned(param_bf16, 8)) return QLORA_ERR_INVALID_VALUE;
  if (!(beta1 >= 0.0f && beta1 < 1.0f) || !(beta2 >= 0.0f && beta2 < 1.0f)) return QLORA_ERR_INVALID_VALUE;
  if (!(eps > 0.0f) || !std::isfinite(eps) || !(lr >= 0.0f) || !std::isfinite(lr)) return QLORA_ERR_INVALID_VALUE;
  if (!(weight_decay >= 0.0f) || !std::isfinite(weight_decay)) return QLORA_ERR_INVALID_VALUE;
  const AdamwArgs a{param, grad, exp_avg, exp_avg_sq, param_bf16, n, step, lr, beta1, beta2, eps, weight_decay};
  return launch_status(launch_adamw(a, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_silu_gate_fwd(const uint16_t *G, const uint16_t *U, int64_t n, uint16_t *H, void *stream) {
  if (!G || !U || !H || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(G, 16) || !aligned(U, 16) || !aligned(H, 16)) return QLORA_ERR_INVALID_VALUE;
  return launch_status(launch_silu_gate_fwd(G, U, n, H, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_silu_gate_bwd(const uint16_t *G, const uint16_t *U, const uint16_t *dH, int64_t n, uint16_t *dG,
                                   uint16_t *dU, void *stream) {
  if (!G || !U || !dH || !dG || !dU || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(G, 16) || !aligned(U, 16) || !aligned(dH, 16) || !aligned(dG, 16) || !aligned(dU, 16))
    return QLORA_ERR_INVALID_VALUE;
  if (dG == dU) return QLORA_ERR_INVALID_VALUE;
  return launch_status(launch_silu_gate_bwd(G, U, dH, n, dG, dU, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_grad_sum(const uint16_t *const *parts, int32_t k, int64_t n, uint16_t *out, void *stream) {
  if (!parts || !out || k < 1 || k > kMaxSumParts || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(out, 16)) return QLORA_ERR_INVALID_VALUE;
  SumParts sp{};
  sp.k = k;
  for (int i = 0; i < k; ++i) {
    if (!parts[i] || !aligned(parts[i], 16)) return QLORA_ERR_INVALID_VALUE;
    sp.p[i] = parts[i];
  }
  return launch_status(launch_grad_sum(sp, n, out, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_stream_probe(int32_t rd, int32_t wr, int32_t depth, int32_t blocks, const void *src, void *dst,
                                  int64_t n_tiles, void *stream) {
  const bool kind = (rd == 1 && wr == 0) || (rd == 4 && wr == 1) || (rd == 1 && wr == 4);
  const bool shape = (depth == 1 || depth == 2 || depth == 4 || depth == 8) && blocks >= 0 && blocks <= (1 << 20);
  if (!kind || !shape || !src || !dst || n_tiles < 1) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(src, 16) || !aligned(dst, 16)) return QLORA_ERR_INVALID_VALUE;
  if (n_tiles > ((int64_t)1 << 40) / 4096) return QLORA_ERR_INVALID_VALUE;  // beyond any device's memory
  return launch_status(
      launch_stream_probe(rd, wr, depth, blocks, src, dst, n_tiles, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_set_timing_events(int32_t kernel, void *start, void *stop) {
  if (kernel < 0 || kernel > 2) return QLORA_ERR_INVALID_VALUE;
  set_timing_events(kernel, reinterpret_cast<hipEvent_t>(start), reinterpret_cast<hipEvent_t>(stop));
  return QLORA_OK;
}

qlora_status_t qlora_workspace_size(qlora_op_t op, int64_t a, int64_t b, int64_t c, int32_t r,
                                    size_t *bytes) {
  if (!bytes) return QLORA_ERR_INVALID_VALUE;
  switch (op) {
    case QLORA_OP_DOUBLE_QUANT:
      if (a < 1) return QLORA_ERR_INVALID_VALUE;
      *bytes = dq_workspace_bytes();
      return QLORA_OK;
    case QLORA_OP_LINEAR_FWD:
    case QLORA_OP_LINEAR_BWD:
      if (a < 1 || b < 64 || c < 64 || r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_INVALID_VALUE;
      *bytes = round256(op == QLORA_OP_LINEAR_FWD ? linear_fwd_workspace(a, b, c, r)
                                                  : linear_bwd_workspace(a, b, c, r));
      return QLORA_OK;
  }
  return QLORA_ERR_INVALID_VALUE;
}

qlora_status_t qlora_quantize_cb(const void *w, qlora_dtype_t w_dtype, int64_t n, qlora_codebook_t codebook,
                                 uint8_t *codes, float *absmax, void *stream) {
  if (!w || !codes || !absmax || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (w_dtype != QLORA_F32 && w_dtype != QLORA_BF16) return QLORA_ERR_INVALID_VALUE;
  if (codebook < 0 || codebook >= kCodebooks) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(w, 16) || !aligned(codes, 4) || !aligned(absmax, 4)) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  return launch_status(launch_quantize(w, w_dtype == QLORA_BF16, n, codes, absmax, *t,
                                       reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_quantize(const void *w, qlora_dtype_t w_dtype, int64_t n, uint8_t *codes,
                              float *absmax, void *stream) {
  return qlora_quantize_cb(w, w_dtype, n, QLORA_CB_NF4, codes, absmax, stream);
}

qlora_status_t qlora_double_quant(const float *absmax, int64_t nblocks, int8_t *qabsmax, float *scale2,
                                  float *mean, void *workspace, size_t ws_bytes, void *stream) {
  if (!absmax || !qabsmax || !scale2 || !mean || !workspace) return QLORA_ERR_INVALID_VALUE;
  if (nblocks < 1 || nblocks >= (int64_t(1) << 32)) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(absmax, 16) || !aligned(qabsmax, 4) || !aligned(scale2, 4) || !aligned(mean, 4) ||
      !aligned(workspace, 256))
    return QLORA_ERR_INVALID_VALUE;
  if (ws_bytes < dq_workspace_bytes()) return QLORA_ERR_INVALID_VALUE;
  return launch_status(launch_double_quant(absmax, nblocks, qabsmax, scale2, mean, workspace,
                                           reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_double_quant_noalloc(const float *absmax, int64_t nblocks, int8_t *qabsmax, float *scale2,
                                          float *mean, void *stream) {
  if (!absmax || !qabsmax || !scale2 || !mean) return QLORA_ERR_INVALID_VALUE;
  if (nblocks < 1 || nblocks >= (int64_t(1) << 32)) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(absmax, 16) || !aligned(qabsmax, 4) || !aligned(scale2, 4) || !aligned(mean, 4))
    return QLORA_ERR_INVALID_VALUE;
  const hipError_t e = launch_double_quant_noalloc(absmax, nblocks, qabsmax, scale2, mean,
                                                   reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorInvalidDevice) return QLORA_ERR_INVALID_VALUE;
  return launch_status(e);
}

qlora_status_t qlora_dequantize_cb(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                                   const float *mean, int64_t n, qlora_codebook_t codebook, void *out,
                                   qlora_dtype_t out_dtype, void *stream) {
  if (!codes || !qabsmax || !scale2 || !mean || !out || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_INVALID_VALUE;
  if (codebook < 0 || codebook >= kCodebooks) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(scale2, 4) || !aligned(mean, 4))
    return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  return launch_status(launch_dequantize(codes, qabsmax, scale2, mean, n, out, out_dtype == QLORA_BF16,
                                         *t, reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_dequantize(const uint8_t *codes, const int8_t *qabsmax, const float *scale2,
                                const float *mean, int64_t n, void *out, qlora_dtype_t out_dtype,
                                void *stream) {
  return qlora_dequantize_cb(codes, qabsmax, scale2, mean, n, QLORA_CB_NF4, out, out_dtype, stream);
}

qlora_status_t qlora_dequantize_nodq(const uint8_t *codes, const float *absmax, int64_t n,
                                     qlora_codebook_t codebook, void *out, qlora_dtype_t out_dtype,
                                     void *stream) {
  if (!codes || !absmax || !out || n < 1) return QLORA_ERR_INVALID_VALUE;
  if (out_dtype != QLORA_F32 && out_dtype != QLORA_BF16) return QLORA_ERR_INVALID_VALUE;
  if (codebook < 0 || codebook >= kCodebooks) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(absmax, 4)) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  return launch_status(launch_dequantize(codes, nullptr, nullptr, nullptr, n, out, out_dtype == QLORA_BF16,
                                         *t, reinterpret_cast<hipStream_t>(stream), absmax));
}

qlora_status_t qlora_codebook_levels(qlora_codebook_t codebook, float *levels) {
  if (!levels || codebook < 0 || codebook >= kCodebooks) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  for (int i = 0; i < 16; ++i) levels[i] = t->level[i];
  return QLORA_OK;
}

qlora_status_t qlora_linear_fwd_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *X,
                                   int64_t M, const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                                   uint16_t *Y, uint16_t *T, void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_weight(W, codebook) || !X || !Y || M < 1 || M > (int64_t(1) << 31)) return QLORA_ERR_INVALID_VALUE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!L1 || !L2 || !T)) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(X, 16) || !aligned(Y, 16)) return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!aligned(L1, 16) || !aligned(L2, 16) || !aligned(T, 16))) return QLORA_ERR_INVALID_VALUE;
  const size_t need = round256(linear_fwd_workspace(M, W->h, W->o, r));
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 256))) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  LinearArgs a{W->codes, W->qabsmax, W->scale2, W->mean, W->h, W->o, M, r, s};
  return launch_status(launch_linear_fwd(a, X, L1, L2, Y, T, workspace, *t,
                                         reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_linear_fwd(const qlora_nf4_weight_t *W, const uint16_t *X, int64_t M,
                                const uint16_t *L1, const uint16_t *L2, int32_t r, float s,
                                uint16_t *Y, uint16_t *T, void *workspace, size_t ws_bytes,
                                void *stream) {
  return qlora_linear_fwd_cb(W, QLORA_CB_NF4, X, M, L1, L2, r, s, Y, T, workspace, ws_bytes, stream);
}

qlora_status_t qlora_linear_bwd_cb(const qlora_nf4_weight_t *W, qlora_codebook_t codebook, const uint16_t *X,
                                   const uint16_t *T, const uint16_t *dY, int64_t M, const uint16_t *L1,
                                   const uint16_t *L2, int32_t r, float s, uint16_t *dX, float *dL1, float *dL2,
                                   void *workspace, size_t ws_bytes, void *stream) {
  if (!valid_weight(W, codebook) || !dY || !dX || M < 1 || M > (int64_t(1) << 31)) return QLORA_ERR_INVALID_VALUE;
  if (r < 0 || r > QLORA_MAX_RANK) return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!X || !T || !L1 || !L2 || !dL1 || !dL2)) return QLORA_ERR_INVALID_VALUE;
  if (!aligned(dY, 16) || !aligned(dX, 16)) return QLORA_ERR_INVALID_VALUE;
  if (r > 0 && (!aligned(X, 16) || !aligned(T, 16) || !aligned(L1, 16) || !aligned(L2, 16) ||
                !aligned(dL1, 16) || !aligned(dL2, 16)))
    return QLORA_ERR_INVALID_VALUE;
  if (!linear_bwd_supported(M, W->h, W->o, r)) return QLORA_ERR_UNSUPPORTED;
  const size_t need = round256(linear_bwd_workspace(M, W->h, W->o, r));
  if (need && (!workspace || ws_bytes < need || !aligned(workspace, 256))) return QLORA_ERR_INVALID_VALUE;
  const Nf4Tables *t = host_tables(codebook);
  if (!t) return QLORA_ERR_INTERNAL;
  LinearArgs a{W->codes, W->qabsmax, W->scale2, W->mean, W->h, W->o, M, r, s};
  return launch_status(launch_linear_bwd(a, X, T, dY, L1, L2, dX, dL1, dL2, workspace, *t,
                                         reinterpret_cast<hipStream_t>(stream)));
}

qlora_status_t qlora_linear_bwd(const qlora_nf4_weight_t *W, const uint16_t *X, const uint16_t *T,
                                const uint16_t *dY, int64_t M, const uint16_t *L1, const uint16_t *L2,
                                int32_t r, float s, uint16_t *dX, float *dL1, float *dL2,
                                void *workspace, size_t ws_bytes, void *stream) {
  return qlora_linear_bwd_cb(W, QLORA_CB_NF4, X, T, dY, M, L1, L2, r, s, dX, dL1, dL2, workspace, ws_bytes, stream);
}

}  // extern "C"
