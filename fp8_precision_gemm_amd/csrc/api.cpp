// C ABI of liblokafp8.so: argument validation, workspace sizing and dispatch
// to the gfx950 kernels.  The contract of each entry point (with the page
// passages it follows) is in include/loka_fp8.h.  Validation runs before any
// HIP call, so every error path is reachable without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/loka_fp8.h"
#include "launch.hpp"

namespace {

thread_local char g_last_error[512] = "";

loka_status fail(loka_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
loka_status fail(loka_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

loka_status hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) {
    g_last_error[0] = '\0';
    return LOKA_OK;
  }
  return fail(LOKA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

#define REQUIRE(cond, st, ...) \
  do {                         \
    if (!(cond)) return fail(st, __VA_ARGS__); \
  } while (0)

#define REQUIRE_ALIGNED(ptr) \
  REQUIRE((ptr) == nullptr || aligned16(ptr), LOKA_ERR_ALIGNMENT, "%s is not 16-byte aligned", #ptr)

loka_status check_workspace(size_t need, const void* ws, size_t have) {
  if (need == 0) return LOKA_OK;
  REQUIRE(ws != nullptr, LOKA_ERR_WORKSPACE, "workspace is NULL but %zu bytes are required", need);
  REQUIRE(have >= need, LOKA_ERR_WORKSPACE, "workspace_bytes %zu < required %zu", have, need);
  REQUIRE(aligned16(ws), LOKA_ERR_ALIGNMENT, "workspace is not 16-byte aligned");
  return LOKA_OK;
}

// Shape checks shared by the forward, backward and grouped entry points.
loka_status check_fwd_shape(int64_t M, int64_t N, int64_t K, int x_mode) {
  REQUIRE(M >= 0 && N >= 0 && K >= 0, LOKA_ERR_INVALID_ARG, "negative size (M=%lld N=%lld K=%lld)", (long long)M,
          (long long)N, (long long)K);
  REQUIRE(N % 64 == 0 && N >= 64 && N <= 1024, LOKA_ERR_UNSUPPORTED,
          "N=%lld: the fused LayerNorm needs N %% 64 == 0 and 64 <= N <= 1024", (long long)N);
  REQUIRE(K >= 16 && K <= 2048 && K % 16 == 0, LOKA_ERR_UNSUPPORTED, "K=%lld: need K %% 16 == 0, 16 <= K <= 2048",
          (long long)K);
  REQUIRE((x_mode != LOKA_SCALE_MX32_ROW && x_mode != LOKA_SCALE_MX32_SQ) || K % 32 == 0, LOKA_ERR_UNSUPPORTED,
          "MX32 needs K %% 32 == 0 (K=%lld)", (long long)K);
  REQUIRE(M <= ((int64_t)1 << 31) - 64, LOKA_ERR_UNSUPPORTED, "M=%lld too large", (long long)M);
  return LOKA_OK;
}

loka_status check_eps(float eps) {
  REQUIRE(std::isfinite(eps) && eps >= 0.0f, LOKA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  return LOKA_OK;
}

}  // namespace

extern "C" {

int loka_abi_version(void) { return LOKA_ABI_VERSION; }

const char* loka_status_string(loka_status s) {
  // a C caller may pass any int: take the value's bytes rather than loading
  // an out-of-range enumerator (undefined in C++)
  int v;
  std::memcpy(&v, &s, sizeof v);
  switch (v) {
    case LOKA_OK: return "LOKA_OK";
    case LOKA_ERR_INVALID_ARG: return "LOKA_ERR_INVALID_ARG";
    case LOKA_ERR_UNSUPPORTED: return "LOKA_ERR_UNSUPPORTED";
    case LOKA_ERR_ALIGNMENT: return "LOKA_ERR_ALIGNMENT";
    case LOKA_ERR_WORKSPACE: return "LOKA_ERR_WORKSPACE";
    case LOKA_ERR_HIP: return "LOKA_ERR_HIP";
  }
  return "LOKA_ERR_UNKNOWN";
}

const char* loka_last_error(void) { return g_last_error; }

// ---------------------------------------------------------------------------
size_t loka_quant_workspace_size(const loka_quant_args* a) {
  if (a == nullptr || a->rows < 0 || a->cols < 0 || a->mode < 0 || a->mode > LOKA_SCALE_MX32_SQ) return 0;
  if (a->rows == 0 || a->cols == 0) return 0;
  return (size_t)loka::quant_plan(a->rows, a->cols, a->mode).ws_floats * sizeof(float);
}

loka_status loka_quant_fp8(const loka_quant_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->rows >= 0 && a->cols >= 0, LOKA_ERR_INVALID_ARG, "negative rows/cols");
  REQUIRE(a->ld >= a->cols, LOKA_ERR_INVALID_ARG, "ld %lld < cols %lld", (long long)a->ld, (long long)a->cols);
  REQUIRE(a->src_dtype == LOKA_DTYPE_BF16 || a->src_dtype == LOKA_DTYPE_F32, LOKA_ERR_INVALID_ARG, "bad src_dtype %d",
          a->src_dtype);
  REQUIRE(a->fmt == LOKA_E4M3 || a->fmt == LOKA_E5M2, LOKA_ERR_INVALID_ARG, "bad fmt %d", a->fmt);
  REQUIRE(a->mode >= LOKA_SCALE_TENSOR && a->mode <= LOKA_SCALE_MX32_SQ, LOKA_ERR_INVALID_ARG, "bad mode %d", a->mode);
  REQUIRE(a->transpose_out >= 0 && a->transpose_out <= 3, LOKA_ERR_INVALID_ARG, "transpose_out must be 0, 1, 2 or 3");
  const bool mx = a->mode == LOKA_SCALE_MX32_ROW || a->mode == LOKA_SCALE_MX32_COL || a->mode == LOKA_SCALE_MX32_SQ;
  REQUIRE(!(mx && a->amax != nullptr), LOKA_ERR_INVALID_ARG, "amax output is not defined for MX modes");
  REQUIRE(a->cols % 16 == 0, LOKA_ERR_UNSUPPORTED, "cols %% 16 != 0");
  REQUIRE(a->ld % 8 == 0, LOKA_ERR_ALIGNMENT, "ld %% 8 != 0");
  REQUIRE(a->mode != LOKA_SCALE_MX32_ROW || a->cols % 32 == 0, LOKA_ERR_UNSUPPORTED, "MX32_ROW needs cols %% 32 == 0");
  REQUIRE(a->mode != LOKA_SCALE_MX32_COL || a->rows % 32 == 0, LOKA_ERR_UNSUPPORTED, "MX32_COL needs rows %% 32 == 0");
  REQUIRE(a->mode != LOKA_SCALE_MX32_SQ || (a->rows % 32 == 0 && a->cols % 32 == 0), LOKA_ERR_UNSUPPORTED,
          "MX32_SQ needs rows %% 32 == 0 and cols %% 32 == 0");
  REQUIRE(!a->transpose_out || a->rows % 16 == 0, LOKA_ERR_UNSUPPORTED, "transpose_out needs rows %% 16 == 0");
  const bool empty = a->rows == 0 || a->cols == 0;
  if (!empty) {
    REQUIRE(a->src && a->codes && a->scales, LOKA_ERR_INVALID_ARG, "src, codes and scales are required");
  }
  REQUIRE_ALIGNED(a->src);
  REQUIRE_ALIGNED(a->codes);
  REQUIRE_ALIGNED(a->scales);
  REQUIRE_ALIGNED(a->amax);
  loka_status st = check_workspace(loka_quant_workspace_size(a), a->workspace, a->workspace_bytes);
  if (st != LOKA_OK) return st;
  if (empty) return LOKA_OK;
  loka::QuantLaunch q{};
  q.src = a->src; q.rows = a->rows; q.cols = a->cols; q.ld = a->ld;
  q.src_dtype = a->src_dtype; q.fmt = a->fmt; q.mode = a->mode; q.transpose_out = a->transpose_out;
  q.codes = a->codes; q.scales = a->scales; q.amax_out = a->amax; q.workspace = a->workspace;
  return hip_status(loka::launch_quant(q, static_cast<hipStream_t>(stream)), "loka_quant_fp8");
}

// ---------------------------------------------------------------------------
size_t loka_gemm_fp8_ln_workspace_size(const loka_fwd_args* a) {
  if (a == nullptr || a->M <= 0 || a->K <= 0) return 0;
  return loka::fwd_workspace_bytes(a->M, a->N, a->K, a->x_mode, (a->flags & LOKA_FWD_W_PACKED) != 0,
                                   (a->flags & LOKA_FWD_BLOCKNORM_HSWISH) != 0);
}

}  // extern "C"

namespace {

// Every check of loka_gemm_fp8_ln except the workspace's.
loka_status validate_fwd(const loka_fwd_args* a) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->x_mode == LOKA_SCALE_TENSOR || a->x_mode == LOKA_SCALE_ROW || a->x_mode == LOKA_SCALE_MX32_ROW ||
              a->x_mode == LOKA_SCALE_MX32_SQ,
          LOKA_ERR_INVALID_ARG, "x_mode must be TENSOR, ROW, MX32_ROW or MX32_SQ (got %d)", a->x_mode);
  REQUIRE((a->flags & ~(LOKA_FWD_W_PACKED | LOKA_FWD_BLOCKNORM_HSWISH)) == 0, LOKA_ERR_INVALID_ARG,
          "unknown flags %d", a->flags);
  const bool packed = (a->flags & LOKA_FWD_W_PACKED) != 0;
  const bool blocknorm = (a->flags & LOKA_FWD_BLOCKNORM_HSWISH) != 0;
  loka_status st;
  if (blocknorm) {
    REQUIRE(a->M >= 0 && a->N >= 0 && a->K >= 0, LOKA_ERR_INVALID_ARG, "negative size");
    REQUIRE(a->x_mode == LOKA_SCALE_ROW, LOKA_ERR_UNSUPPORTED, "the BlockNorm epilogue supports x_mode ROW only");
    REQUIRE(loka::fwd_blocknorm_fits(a->N, a->K), LOKA_ERR_UNSUPPORTED,
            "BlockNorm needs N %% 256 == 0, 256 <= N <= 8192, K %% 16 == 0, 16 <= K <= 1024 (got N=%lld K=%lld)",
            (long long)a->N, (long long)a->K);
    REQUIRE(a->M <= ((int64_t)1 << 31) - 64, LOKA_ERR_UNSUPPORTED, "M too large");
    REQUIRE(a->gamma == nullptr && a->beta == nullptr && a->mean == nullptr && a->rstd == nullptr,
            LOKA_ERR_INVALID_ARG, "the BlockNorm epilogue has no gamma/beta and no mean/rstd outputs");
  } else {
    if ((st = check_fwd_shape(a->M, a->N, a->K, a->x_mode)) != LOKA_OK) return st;
  }
  REQUIRE(!packed || blocknorm || loka::fwd_weight_resident(a->N, a->K), LOKA_ERR_UNSUPPORTED,
          "LOKA_FWD_W_PACKED needs the weight-resident shapes: N <= 512 and K <= 1024 (N <= 256), 640 (N <= 384) "
          "or 512 (N <= 512); got N=%lld K=%lld",
          (long long)a->N, (long long)a->K);
  if (a->x_mode == LOKA_SCALE_MX32_SQ) {
    REQUIRE(!blocknorm, LOKA_ERR_UNSUPPORTED, "the BlockNorm epilogue supports x_mode ROW only");
    REQUIRE(a->M % 32 == 0 && a->N % 32 == 0, LOKA_ERR_UNSUPPORTED, "MX32_SQ needs M %% 32 == 0 (M=%lld)",
            (long long)a->M);
    REQUIRE(loka::fwd_weight_resident(a->N, a->K), LOKA_ERR_UNSUPPORTED,
            "MX32_SQ runs on the weight-resident shapes: N <= 512 and K <= 1024 (N <= 256), 640 (N <= 384) or 512 "
            "(N <= 512); got N=%lld K=%lld",
            (long long)a->N, (long long)a->K);
    REQUIRE(a->qx_out == nullptr && a->sx_out == nullptr, LOKA_ERR_INVALID_ARG,
            "MX32_SQ takes X quantized: qx_out and sx_out must be NULL");
    if (a->M > 0) REQUIRE(a->x_scales != nullptr, LOKA_ERR_INVALID_ARG, "MX32_SQ needs x_scales");
  } else {
    REQUIRE(a->x_scales == nullptr, LOKA_ERR_INVALID_ARG, "x_scales is only for x_mode MX32_SQ");
  }
  if (a->y_codes != nullptr || a->y_scales != nullptr) {
    REQUIRE(a->y_codes != nullptr && a->y_scales != nullptr, LOKA_ERR_INVALID_ARG,
            "y_codes and y_scales go together");
    REQUIRE(!blocknorm && (a->N == 256 || a->N == 512) && loka::fwd_weight_resident(a->N, a->K) && a->M % 32 == 0,
            LOKA_ERR_UNSUPPORTED,
            "the square-block Y output needs the LayerNorm epilogue, N = 256 or 512, the weight-resident shapes and "
            "M %% 32 == 0 (got M=%lld N=%lld K=%lld)",
            (long long)a->M, (long long)a->N, (long long)a->K);
  }
  if ((st = check_eps(a->eps)) != LOKA_OK) return st;
  if (a->M > 0) REQUIRE(a->x && a->qw && a->sw && a->y, LOKA_ERR_INVALID_ARG, "x, qw, sw and y are required");
  REQUIRE_ALIGNED(a->x); REQUIRE_ALIGNED(a->qw); REQUIRE_ALIGNED(a->sw); REQUIRE_ALIGNED(a->bias);
  REQUIRE_ALIGNED(a->gamma); REQUIRE_ALIGNED(a->beta); REQUIRE_ALIGNED(a->y); REQUIRE_ALIGNED(a->z);
  REQUIRE_ALIGNED(a->mean); REQUIRE_ALIGNED(a->rstd); REQUIRE_ALIGNED(a->qx_out); REQUIRE_ALIGNED(a->sx_out);
  return LOKA_OK;
}

loka::FwdLaunch fwd_launch(const loka_fwd_args* a, void* workspace) {
  loka::FwdLaunch f{};
  f.M = a->M; f.N = a->N; f.K = a->K; f.x_mode = a->x_mode; f.eps = a->eps;
  f.x = a->x; f.qw = a->qw; f.sw = a->sw; f.bias = a->bias; f.gamma = a->gamma; f.beta = a->beta;
  f.y = a->y; f.z = a->z; f.mean = a->mean; f.rstd = a->rstd; f.qx_out = a->qx_out; f.sx_out = a->sx_out;
  f.workspace = workspace;
  f.x_scales = a->x_scales;
  f.y_codes = a->y_codes;
  f.y_scales = a->y_scales;
  f.w_packed = (a->flags & LOKA_FWD_W_PACKED) != 0;
  f.blocknorm = (a->flags & LOKA_FWD_BLOCKNORM_HSWISH) != 0;
  return f;
}

}  // namespace

extern "C" {

loka_status loka_gemm_fp8_ln(const loka_fwd_args* a, void* stream) {
  loka_status st = validate_fwd(a);
  if (st != LOKA_OK) return st;
  if ((st = check_workspace(loka_gemm_fp8_ln_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK) return st;
  if (a->M == 0) return LOKA_OK;
  return hip_status(loka::launch_fwd(fwd_launch(a, a->workspace), static_cast<hipStream_t>(stream)),
                    "loka_gemm_fp8_ln");
}

loka_status loka_gemm_fp8_ln_noalloc(const loka_fwd_args* a, void* stream) {
  loka_status st = validate_fwd(a);
  if (st != LOKA_OK) return st;
  const size_t need = loka_gemm_fp8_ln_workspace_size(a);
  REQUIRE(need <= loka::noalloc_scratch_bytes(), LOKA_ERR_UNSUPPORTED,
          "this call needs %zu bytes of scratch; loka_gemm_fp8_ln_noalloc holds %zu (use loka_gemm_fp8_ln with a "
          "workspace, or LOKA_FWD_W_PACKED)",
          need, loka::noalloc_scratch_bytes());
  if (a->M == 0) return LOKA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  hipError_t e = loka::noalloc_scratch(s, &scratch);
  if (e != hipSuccess) return hip_status(e, "loka_gemm_fp8_ln_noalloc (device scratch)");
  return hip_status(loka::launch_fwd(fwd_launch(a, scratch), s), "loka_gemm_fp8_ln_noalloc");
}

// ---------------------------------------------------------------------------
size_t loka_gemm_fp8_bwd_workspace_size(const loka_bwd_args* a) {
  if (a == nullptr || a->M <= 0 || a->N <= 0 || a->K <= 0) return 0;
  return loka::bwd_workspace_bytes(a->M, a->N, a->K, (a->flags & LOKA_BWD_MX32_SQ) != 0);
}

loka_status loka_gemm_fp8_bwd(const loka_bwd_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE((a->flags & ~(LOKA_BWD_NO_LN | LOKA_BWD_MX32_SQ | LOKA_BWD_W_PACKED)) == 0, LOKA_ERR_INVALID_ARG,
          "unknown flags %d", a->flags);
  const bool sq = (a->flags & LOKA_BWD_MX32_SQ) != 0;
  const bool w_packed = (a->flags & LOKA_BWD_W_PACKED) != 0;
  REQUIRE(!(sq && w_packed && a->M > 0 && !a->qw_row), LOKA_ERR_INVALID_ARG,
          "LOKA_BWD_MX32_SQ with LOKA_BWD_W_PACKED needs qw_row (the packed dgrad weight)");
  REQUIRE(!sq || (!a->xc_codes && !a->xc_scales && !a->dzc_codes && !a->dzc_scales), LOKA_ERR_INVALID_ARG,
          "the column-code outputs belong to the ROW recipe");
  loka_status st = check_fwd_shape(a->M, a->N, a->K, sq ? LOKA_SCALE_MX32_SQ : LOKA_SCALE_ROW);
  if (st != LOKA_OK) return st;
  REQUIRE(a->K % 64 == 0 && a->K <= 1024, LOKA_ERR_UNSUPPORTED, "backward needs K %% 64 == 0 and K <= 1024");
  REQUIRE(a->M % 16 == 0, LOKA_ERR_UNSUPPORTED, "backward needs M %% 16 == 0");
  if (sq)
    REQUIRE(a->M % 32 == 0 && a->N <= 512 && a->K <= 512, LOKA_ERR_UNSUPPORTED,
            "the square-block backward needs M %% 32 == 0, N <= 512 and K <= 512 (got M=%lld N=%lld K=%lld)",
            (long long)a->M, (long long)a->N, (long long)a->K);
  const bool no_ln = (a->flags & LOKA_BWD_NO_LN) != 0;
  if (a->M > 0) {
    if (sq) {
      REQUIRE(a->dy && a->qx && a->sx && a->qw && a->sw && a->dx && a->dw, LOKA_ERR_INVALID_ARG,
              "dy, qx, sx, qw, sw, dx and dw are required");
      if (!no_ln)
        REQUIRE(a->mean && a->rstd, LOKA_ERR_INVALID_ARG, "the forward's mean and rstd are required");
    } else {
      REQUIRE(a->dy && a->x && a->qw_row && a->sw_row && a->dx && a->dw, LOKA_ERR_INVALID_ARG,
              "dy, x, qw_row, sw_row, dx and dw are required");
      if (!no_ln)
        REQUIRE(a->qx && a->sx && a->mean && a->rstd && a->qw && a->sw, LOKA_ERR_INVALID_ARG,
                "the forward context (qx, sx, mean, rstd, qw, sw) is required");
    }
  }
  REQUIRE(!(no_ln && (a->dgamma || a->dbeta)), LOKA_ERR_INVALID_ARG, "dgamma/dbeta are undefined without LayerNorm");
  REQUIRE_ALIGNED(a->dy); REQUIRE_ALIGNED(a->qx); REQUIRE_ALIGNED(a->sx); REQUIRE_ALIGNED(a->mean);
  REQUIRE_ALIGNED(a->rstd); REQUIRE_ALIGNED(a->qw); REQUIRE_ALIGNED(a->sw); REQUIRE_ALIGNED(a->bias);
  REQUIRE_ALIGNED(a->gamma); REQUIRE_ALIGNED(a->x); REQUIRE_ALIGNED(a->qw_row); REQUIRE_ALIGNED(a->sw_row);
  REQUIRE_ALIGNED(a->dx); REQUIRE_ALIGNED(a->dw); REQUIRE_ALIGNED(a->dgamma); REQUIRE_ALIGNED(a->dbeta);
  REQUIRE_ALIGNED(a->dbias); REQUIRE_ALIGNED(a->dz); REQUIRE_ALIGNED(a->dz_codes); REQUIRE_ALIGNED(a->dz_scales);
  REQUIRE_ALIGNED(a->xc_codes); REQUIRE_ALIGNED(a->xc_scales); REQUIRE_ALIGNED(a->dzc_codes);
  REQUIRE_ALIGNED(a->dzc_scales);
  if ((st = check_workspace(loka_gemm_fp8_bwd_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK)
    return st;
  if (a->M == 0) return LOKA_OK;
  loka::BwdLaunch b{};
  b.M = a->M; b.N = a->N; b.K = a->K; b.no_ln = no_ln ? 1 : 0; b.sq = sq;
  b.dy = a->dy; b.qx = a->qx; b.sx = a->sx; b.mean = a->mean; b.rstd = a->rstd; b.qw = a->qw; b.sw = a->sw;
  b.bias = a->bias; b.gamma = a->gamma; b.x = a->x; b.qw_row = a->qw_row; b.sw_row = a->sw_row;
  b.dx = a->dx; b.dw = a->dw; b.dgamma = a->dgamma; b.dbeta = a->dbeta; b.dbias = a->dbias;
  b.dz = a->dz; b.dz_codes = a->dz_codes; b.dz_scales = a->dz_scales; b.workspace = a->workspace;
  b.w_packed = w_packed;
  b.xc_codes = a->xc_codes; b.xc_scales = a->xc_scales; b.dzc_codes = a->dzc_codes; b.dzc_scales = a->dzc_scales;
  return hip_status(loka::launch_bwd(b, static_cast<hipStream_t>(stream)), "loka_gemm_fp8_bwd");
}

// ---------------------------------------------------------------------------
size_t loka_mere_workspace_size(const loka_mere_args* a) {
  if (a == nullptr || a->S <= 0) return 0;
  return loka::mere_workspace_bytes(a->S);
}

loka_status loka_mere_z(const loka_mere_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->M >= 1 && a->N >= 1 && a->K >= 1 && a->S >= 1, LOKA_ERR_INVALID_ARG, "M, N, K and S must be >= 1");
  REQUIRE(a->K <= loka::mere_max_k() && a->N <= 8192, LOKA_ERR_UNSUPPORTED, "MERE needs K <= %d and N <= 8192",
          loka::mere_max_k());
  REQUIRE(a->x && a->w && a->z && a->rows && a->out, LOKA_ERR_INVALID_ARG, "x, w, z, rows and out are required");
  REQUIRE_ALIGNED(a->x); REQUIRE_ALIGNED(a->w); REQUIRE_ALIGNED(a->bias); REQUIRE_ALIGNED(a->z);
  REQUIRE_ALIGNED(a->rows); REQUIRE_ALIGNED(a->out);
  loka_status st;
  if ((st = check_workspace(loka_mere_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK) return st;
  loka::MereLaunch m{a->M, a->N, a->K, a->S, a->x, a->w, a->bias, a->z, a->rows, a->out, a->workspace};
  return hip_status(loka::launch_mere(m, static_cast<hipStream_t>(stream)), "loka_mere_z");
}

// ---------------------------------------------------------------------------
namespace {
constexpr int64_t kProbeMaxDim = 2048;
bool probe_dim_ok(int64_t d) { return d >= 1 && d <= kProbeMaxDim; }
}  // namespace

size_t loka_probe_input_workspace_size(const loka_probe_input_args* a) {
  if (a == nullptr || a->B < 1 || !probe_dim_ok(a->K)) return 0;
  return loka::probe_input_ws(a->B, a->K);
}
loka_status loka_probe_input_update(const loka_probe_input_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->B >= 1 && a->n_old >= 0, LOKA_ERR_INVALID_ARG, "B >= 1 and n_old >= 0 are required");
  REQUIRE(probe_dim_ok(a->K), LOKA_ERR_UNSUPPORTED, "the Probe needs 1 <= K <= %lld", (long long)kProbeMaxDim);
  REQUIRE(a->T && a->mu && a->S, LOKA_ERR_INVALID_ARG, "T, mu and S are required");
  REQUIRE_ALIGNED(a->T); REQUIRE_ALIGNED(a->mu); REQUIRE_ALIGNED(a->S);
  loka_status st;
  if ((st = check_workspace(loka_probe_input_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK)
    return st;
  loka::ProbeInputLaunch l{a->B, a->K, a->n_old, a->T, a->mu, a->S, a->workspace};
  return hip_status(loka::probe_input_update(l, static_cast<hipStream_t>(stream)), "loka_probe_input_update");
}

size_t loka_probe_weight_workspace_size(const loka_probe_weight_args* a) {
  if (a == nullptr || !probe_dim_ok(a->R) || !probe_dim_ok(a->C) || a->first) return 0;
  return loka::probe_weight_ws(a->R, a->C);
}
loka_status loka_probe_weight_update(const loka_probe_weight_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(probe_dim_ok(a->R) && probe_dim_ok(a->C), LOKA_ERR_UNSUPPORTED, "the Probe needs 1 <= R, C <= %lld",
          (long long)kProbeMaxDim);
  REQUIRE(std::isfinite(a->m) && a->m >= 0.0f && a->m < 1.0f, LOKA_ERR_INVALID_ARG, "momentum must be in [0, 1)");
  REQUIRE(a->W && a->M && a->U && a->V && (a->first || a->info), LOKA_ERR_INVALID_ARG,
          "W, M, U, V (and info unless first) are required");
  REQUIRE_ALIGNED(a->W); REQUIRE_ALIGNED(a->M); REQUIRE_ALIGNED(a->U); REQUIRE_ALIGNED(a->V);
  loka_status st;
  if ((st = check_workspace(loka_probe_weight_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK)
    return st;
  loka::ProbeWeightLaunch l{a->R, a->C, a->m, a->first != 0, a->W, a->M, a->U, a->V, a->info, a->workspace};
  return hip_status(loka::probe_weight_update(l, static_cast<hipStream_t>(stream)), "loka_probe_weight_update");
}

size_t loka_probe_sample_input_workspace_size(const loka_probe_sample_input_args* a) {
  if (a == nullptr || a->B < 1 || !probe_dim_ok(a->K)) return 0;
  return loka::probe_sample_input_ws(a->B, a->K);
}
loka_status loka_probe_sample_input(const loka_probe_sample_input_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->B >= 1 && a->n >= 2, LOKA_ERR_INVALID_ARG, "B >= 1 and n >= 2 are required");
  REQUIRE(probe_dim_ok(a->K), LOKA_ERR_UNSUPPORTED, "the Probe needs 1 <= K <= %lld", (long long)kProbeMaxDim);
  REQUIRE(a->mu && a->S && a->out && a->info, LOKA_ERR_INVALID_ARG, "mu, S, out and info are required");
  REQUIRE_ALIGNED(a->mu); REQUIRE_ALIGNED(a->S); REQUIRE_ALIGNED(a->out);
  loka_status st;
  if ((st = check_workspace(loka_probe_sample_input_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK)
    return st;
  loka::ProbeSampleInputLaunch l{a->B, a->K, a->n, a->mu, a->S, a->seed, a->out, a->info, a->workspace};
  return hip_status(loka::probe_sample_input(l, static_cast<hipStream_t>(stream)), "loka_probe_sample_input");
}

size_t loka_probe_sample_weight_workspace_size(const loka_probe_sample_weight_args* a) {
  if (a == nullptr || !probe_dim_ok(a->R) || !probe_dim_ok(a->C)) return 0;
  return loka::probe_sample_weight_ws(a->R, a->C);
}
loka_status loka_probe_sample_weight(const loka_probe_sample_weight_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(probe_dim_ok(a->R) && probe_dim_ok(a->C), LOKA_ERR_UNSUPPORTED, "the Probe needs 1 <= R, C <= %lld",
          (long long)kProbeMaxDim);
  REQUIRE(a->M && a->U && a->V && a->out && a->info, LOKA_ERR_INVALID_ARG, "M, U, V, out and info are required");
  REQUIRE_ALIGNED(a->M); REQUIRE_ALIGNED(a->U); REQUIRE_ALIGNED(a->V); REQUIRE_ALIGNED(a->out);
  loka_status st;
  if ((st = check_workspace(loka_probe_sample_weight_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK)
    return st;
  loka::ProbeSampleWeightLaunch l{a->R, a->C, a->M, a->U, a->V, a->seed, a->out, a->info, a->workspace};
  return hip_status(loka::probe_sample_weight(l, static_cast<hipStream_t>(stream)), "loka_probe_sample_weight");
}

// The pages' rule, step by step: the accuracy filter, the speed filter, then
// the shortest time among what passes.
loka_status loka_dispatch_select(const loka_dispatch_candidate* c, int32_t n, double baseline_us, double mere_max,
                                 double min_speedup, int32_t* choice) {
  REQUIRE(choice != nullptr, LOKA_ERR_INVALID_ARG, "choice is NULL");
  REQUIRE(n >= 0 && (n == 0 || c != nullptr), LOKA_ERR_INVALID_ARG, "bad candidate array");
  REQUIRE(std::isfinite(baseline_us) && baseline_us > 0.0, LOKA_ERR_INVALID_ARG, "baseline_us must be finite, > 0");
  REQUIRE(std::isfinite(mere_max) && mere_max > 0.0 && std::isfinite(min_speedup) && min_speedup > 0.0,
          LOKA_ERR_INVALID_ARG, "thresholds must be finite and > 0");
  int32_t best = -1;
  double best_us = 0.0;
  for (int32_t i = 0; i < n; ++i) {
    const double us = c[i].us, e = c[i].mere;
    if (!std::isfinite(us) || !std::isfinite(e) || us <= 0.0) continue;
    if (!(e < mere_max)) continue;                  // accuracy
    if (!(baseline_us / us > min_speedup)) continue;  // speed
    if (best < 0 || us < best_us) {
      best = i;
      best_us = us;
    }
  }
  *choice = best;
  return LOKA_OK;
}

// ---------------------------------------------------------------------------
static_assert(sizeof(loka_group_desc) == sizeof(loka::GroupDev), "group descriptor layouts differ");

size_t loka_grouped_workspace_size(const loka_grouped_args* a) {
  if (a == nullptr || a->num_groups <= 0) return 0;
  return loka::grouped_workspace_bytes(a->num_groups, reinterpret_cast<const loka::GroupDev*>(a->groups),
                                       (a->flags & LOKA_FWD_W_PACKED) != 0);
}

loka_status loka_grouped_gemm_fp8_ln(const loka_grouped_args* a, void* stream) {
  REQUIRE(a != nullptr, LOKA_ERR_INVALID_ARG, "args is NULL");
  REQUIRE(a->num_groups >= 0, LOKA_ERR_INVALID_ARG, "num_groups < 0");
  REQUIRE(a->x_mode == LOKA_SCALE_ROW, LOKA_ERR_UNSUPPORTED, "grouped launch supports x_mode ROW only");
  REQUIRE((a->flags & ~LOKA_FWD_W_PACKED) == 0, LOKA_ERR_INVALID_ARG, "unknown flags %d", a->flags);
  loka_status st = check_eps(a->eps);
  if (st != LOKA_OK) return st;
  if (a->num_groups == 0) return LOKA_OK;
  REQUIRE(a->groups != nullptr, LOKA_ERR_INVALID_ARG, "groups is NULL");
  REQUIRE(a->num_groups <= loka::grouped_max_groups(), LOKA_ERR_UNSUPPORTED, "num_groups %d > %d", a->num_groups,
          loka::grouped_max_groups());
  int64_t tiles = 0;
  for (int i = 0; i < a->num_groups; ++i) {
    const loka_group_desc& g = a->groups[i];
    st = check_fwd_shape(g.M, g.N, g.K, LOKA_SCALE_ROW);
    if (st != LOKA_OK) return fail(st, "group %d: %s", i, std::string(g_last_error).c_str());
    REQUIRE(loka::fwd_weight_resident(g.N, g.K), LOKA_ERR_UNSUPPORTED,
            "group %d: the grouped launch needs N <= 512 and K <= 1024 (N <= 256), 640 (N <= 384) or 512 "
            "(N <= 512); got N=%lld K=%lld",
            i, (long long)g.N, (long long)g.K);
    if (g.M > 0)
      REQUIRE(g.x && g.qw && g.sw && g.y, LOKA_ERR_INVALID_ARG, "group %d: x, qw, sw and y are required", i);
    REQUIRE(aligned16(g.x) && aligned16(g.qw) && aligned16(g.sw) && aligned16(g.bias) && aligned16(g.gamma) &&
                aligned16(g.beta) && aligned16(g.y) && aligned16(g.z),
            LOKA_ERR_ALIGNMENT, "group %d: a pointer is not 16-byte aligned", i);
    tiles += (g.M + 15) / 16;
  }
  REQUIRE(tiles < ((int64_t)1 << 31), LOKA_ERR_UNSUPPORTED, "too many tiles");
  if ((st = check_workspace(loka_grouped_workspace_size(a), a->workspace, a->workspace_bytes)) != LOKA_OK) return st;
  loka::GroupedLaunch gl{};
  gl.num_groups = a->num_groups;
  gl.eps = a->eps;
  gl.groups = reinterpret_cast<const loka::GroupDev*>(a->groups);
  gl.workspace = a->workspace;
  gl.w_packed = (a->flags & LOKA_FWD_W_PACKED) != 0;
  return hip_status(loka::launch_grouped(gl, static_cast<hipStream_t>(stream)), "loka_grouped_gemm_fp8_ln");
}

}  // extern "C"
