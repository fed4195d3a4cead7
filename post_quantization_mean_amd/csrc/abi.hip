// Host side of the C ABI declared in include/awq.h: argument checks (all before any HIP call),
// workspace sizing, and the composition of the search from its steps. No allocation happens
// here; every buffer belongs to the caller.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "awq.h"
#include "internal.h"
#include "variants.h"
#include "w4a16.h"
#include "block.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return AWQ_OK;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(AWQ_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

size_t esize(int dtype) { return dtype == AWQ_DTYPE_BF16 ? 2 : 4; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// byte offsets inside a 256-row tile, up to its end, are signed 32-bit in the error GEMM's
// buffer descriptors
constexpr int64_t kMaxTileBytes = ((int64_t)1 << 31) - 1;

int check_dtype(int dtype) {
  if (dtype != AWQ_DTYPE_BF16 && dtype != AWQ_DTYPE_F32)
    return fail(AWQ_ERR_UNSUPPORTED, "dtype %d is neither AWQ_DTYPE_F32 nor AWQ_DTYPE_BF16", dtype);
  return AWQ_OK;
}

int check_group(int group_size, int64_t d_in) {
  if (group_size != AWQ_GROUP_SIZE)
    return fail(AWQ_ERR_UNSUPPORTED, "group_size %d: only %d is implemented", group_size, AWQ_GROUP_SIZE);
  if (d_in <= 0 || d_in % group_size)
    return fail(AWQ_ERR_SHAPE, "d_in %lld is not a positive multiple of group_size %d", (long long)d_in,
                group_size);
  return AWQ_OK;
}

int check_x(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x) {
  if (n_tokens < 0) return fail(AWQ_ERR_SHAPE, "n_tokens %lld < 0", (long long)n_tokens);
  if (n_tokens == 0) return fail(AWQ_ERR_NO_TOKENS, "n_tokens == 0: no activation mean");
  if (!x) return fail(AWQ_ERR_NULL, "x is NULL");
  if (ld_x < d_in) return fail(AWQ_ERR_ARG, "ld_x %lld < d_in %lld", (long long)ld_x, (long long)d_in);
  if (ld_x % (16 / (int64_t)esize(dtype)))  // the row pitch in bytes is a multiple of 16 (no product: ld_x may be huge)
    return fail(AWQ_ERR_UNSUPPORTED, "ld_x * element size must be a multiple of 16 bytes");
  if (!aligned(x, 16)) return fail(AWQ_ERR_UNSUPPORTED, "x is not 16-byte aligned");
  if (ld_x > kMaxTileBytes || (int64_t)awq::kTileM * ld_x * (int64_t)esize(dtype) > kMaxTileBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "ld_x %lld too large for 32-bit tile offsets", (long long)ld_x);
  return AWQ_OK;
}

int make_parts(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype, int64_t d_in,
               awq::WParts* out) {
  if (!w_parts || !part_rows) return fail(AWQ_ERR_NULL, "w_parts or part_rows is NULL");
  if (n_parts < 1 || n_parts > AWQ_MAX_PARTS)
    return fail(AWQ_ERR_ARG, "n_parts %d outside [1, %d]", n_parts, AWQ_MAX_PARTS);
  memset(out, 0, sizeof *out);
  out->n = n_parts;
  int64_t rows = 0;
  for (int p = 0; p < n_parts; ++p) {
    if (!w_parts[p]) return fail(AWQ_ERR_NULL, "w_parts[%d] is NULL", p);
    if (!aligned(w_parts[p], 16)) return fail(AWQ_ERR_UNSUPPORTED, "w_parts[%d] is not 16-byte aligned", p);
    if (part_rows[p] <= 0) return fail(AWQ_ERR_SHAPE, "part_rows[%d] = %lld must be > 0", p, (long long)part_rows[p]);
    out->ptr[p] = w_parts[p];
    out->row_begin[p] = rows;
    rows += part_rows[p];
  }
  for (int p = n_parts; p <= AWQ_MAX_PARTS; ++p) out->row_begin[p] = rows;
  if (rows > ((int64_t)65535 * 128)) return fail(AWQ_ERR_UNSUPPORTED, "d_out %lld too large", (long long)rows);
  // parts that lie back to back in memory (row slices of one stacked matrix) are one matrix to
  // the kernels, which then skip the per-row part lookup
  bool contiguous = true;
  const int64_t row_bytes = d_in * esize(dtype);
  for (int p = 1; p < n_parts; ++p)
    contiguous = contiguous && (const char*)w_parts[p] == (const char*)w_parts[0] + out->row_begin[p] * row_bytes;
  if (contiguous && n_parts > 1) {
    out->n = 1;
    for (int p = 1; p <= AWQ_MAX_PARTS; ++p) {
      if (p < AWQ_MAX_PARTS) out->ptr[p] = nullptr;
      out->row_begin[p] = rows;
    }
  }
  return AWQ_OK;
}

int check_d_in_bytes(int dtype, int64_t d_in) {
  if (d_in > kMaxTileBytes || (int64_t)awq::kTileN * d_in * (int64_t)esize(dtype) > kMaxTileBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "d_in %lld too large for 32-bit tile offsets", (long long)d_in);
  if (d_in / AWQ_GROUP_SIZE > 65535) return fail(AWQ_ERR_UNSUPPORTED, "d_in %lld too large", (long long)d_in);
  return AWQ_OK;
}

#define TRY(expr)              \
  do {                         \
    int _s = (expr);           \
    if (_s != AWQ_OK) return _s; \
  } while (0)

int check_ratios(const double* ratios, int n_ratios, int formula, const double* w_mean, awq::RatioList* out) {
  if (formula != AWQ_FORMULA_MSMODELSLIM && formula != AWQ_FORMULA_RMS && formula != AWQ_FORMULA_DUO)
    return fail(AWQ_ERR_ARG, "formula %d is not an awq_formula", formula);
  if (formula == AWQ_FORMULA_DUO && !w_mean) return fail(AWQ_ERR_NULL, "AWQ_FORMULA_DUO needs w_mean");
  if (!ratios) return fail(AWQ_ERR_NULL, "ratios is NULL");
  if (n_ratios < 1 || n_ratios > AWQ_MAX_RATIOS)
    return fail(AWQ_ERR_ARG, "n_ratios %d outside [1, %d]", n_ratios, AWQ_MAX_RATIOS);
  memset(out, 0, sizeof *out);
  for (int k = 0; k < n_ratios; ++k) {
    if (!(ratios[k] >= 0.0 && ratios[k] <= 1.0))
      return fail(AWQ_ERR_ARG, "ratios[%d] = %g is outside [0, 1]", k, ratios[k]);
    out->r[k] = ratios[k];
  }
  return AWQ_OK;
}

int check_quantizer(int quantizer) {
  if (quantizer != AWQ_QUANT_INT4_GROUP && quantizer != AWQ_QUANT_INT4_ROW && quantizer != AWQ_QUANT_INT8_ROW_SYM)
    return fail(AWQ_ERR_ARG, "quantizer %d is not an awq_quantizer", quantizer);
  return AWQ_OK;
}

// The search composed from its steps. `ratios` == nullptr selects the msModelSlim grid
// k / n_grid with the main quantizer; otherwise the variant formula and quantizer.
// The Gram form of the loss (gram.hip): worth it when forming G = X^T X once plus one quadratic
// form per ratio costs well under the direct n_grid N x d_in x d_out products. G's symmetry halves
// both: its 256-tiles on and above the diagonal, and per ratio the blocks of G on and above it, about
// d_in (d_in + 256) (N + n_grid d_out) flops in all, against 2 N d_in d_out n_grid. bfloat16
// activations only (G's products are exact there); it needs N >= d_in (the tiles then fit the loss
// layout), and the 32-bit tile offsets bound the padded token count.
bool gram_form(int dtype, int64_t n_tokens, int64_t d_in, int64_t d_out, int n_grid) {
  if (dtype != AWQ_DTYPE_BF16 || n_tokens < d_in || d_in <= 0 || d_out <= 0 || n_grid < 1) return false;
  const int64_t n_pad = awq::gram_n_pad(n_tokens);
  if ((int64_t)awq::kTileM * n_pad * 2 > 0x7FFFFFFF) return false;
  const double direct = 2.0 * (double)n_tokens * (double)d_in * (double)d_out * n_grid;
  const double gram = (double)d_in * ((double)d_in + awq::kTileM) * ((double)n_pad + (double)d_out * n_grid);
  return gram < 0.85 * direct;
}
size_t gram_ws_bytes(int64_t n_tokens, int64_t d_in) {
  const int64_t n_pad = awq::gram_n_pad(n_tokens);
  return round_up((size_t)d_in * (size_t)n_pad * 2, 256) + round_up((size_t)d_in * (size_t)d_in * 4, 256);
}
// the Gram search's buffers beyond delta and tile_sse: float16 G, the exponents, gram_ws_bytes
size_t gram_search_extra(int64_t n_tokens, int64_t d_in, int cand_per_pass) {
  return round_up((size_t)d_in * (size_t)d_in * 2, 256) + 256 + round_up(((size_t)cand_per_pass + 1) * 4, 256) +
         gram_ws_bytes(n_tokens, d_in);
}

int run_search(const void* x, int64_t ld_x, const void* const* w_parts, const int64_t* part_rows, int n_parts,
               int dtype, int64_t n_tokens, int64_t d_in, const double* act_mean, const double* w_mean,
               const double* ratios, int formula, int quantizer, int n_grid, int cand_per_pass,
               double* cand_scales, double* losses, double* best_scales, int32_t* best_info, void* workspace,
               size_t workspace_bytes, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  TRY(check_x(x, dtype, n_tokens, d_in, ld_x));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  const int64_t d_out = w.row_begin[w.n];
  if (!act_mean || !cand_scales || !losses || !best_scales || !best_info)
    return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(cand_scales, 16)) return fail(AWQ_ERR_UNSUPPORTED, "cand_scales is not 16-byte aligned");
  awq::RatioList rl;
  if (ratios) {
    TRY(check_ratios(ratios, n_grid, formula, w_mean, &rl));
    TRY(check_quantizer(quantizer));
  } else if (n_grid < 1 || n_grid > 65535) {
    return fail(AWQ_ERR_ARG, "n_grid %d outside [1, 65535]", n_grid);
  }
  if (cand_per_pass < 1 || cand_per_pass > n_grid)
    return fail(AWQ_ERR_ARG, "cand_per_pass %d outside [1, n_grid]", cand_per_pass);
  const int64_t tiles = awq_error_tiles(n_tokens, d_out);
  if (tiles * cand_per_pass > 0x7FFFFFFF)
    return fail(AWQ_ERR_UNSUPPORTED, "too many tiles for one launch; lower cand_per_pass");
  const size_t need =
      awq_search_workspace_bytes(dtype, n_tokens, d_in, d_out, AWQ_GROUP_SIZE, n_grid, cand_per_pass);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  void* delta = ws;
  double* tile_sse = reinterpret_cast<double*>(
      ws + round_up((size_t)cand_per_pass * (size_t)d_out * (size_t)d_in * esize(dtype), 256));

  hipError_t e = ratios ? awq::launch_candidate_scales_ex(act_mean, w_mean, d_in, rl, n_grid, formula, cand_scales, st)
                        : awq::launch_candidate_scales(act_mean, d_in, n_grid, cand_scales, st);
  if (e != hipSuccess) return hip_fail(e, "candidate_scales launch");
  if (gram_form(dtype, n_tokens, d_in, d_out, n_grid)) {
    // the loss as the quadratic form of G = X^T X (float16 G and delta, power-of-two scales)
    const double bound_b = quantizer == AWQ_QUANT_INT8_ROW_SYM ? 1.27e-6 : 1e-8;  // |delta|'s bound
    char* p = ws + round_up((size_t)cand_per_pass * (size_t)d_out * (size_t)d_in * esize(dtype), 256) +
              round_up((size_t)n_grid * (size_t)tiles * sizeof(double), 256);
    uint16_t* g16 = reinterpret_cast<uint16_t*>(p);
    p += round_up((size_t)d_in * (size_t)d_in * 2, 256);
    int32_t* gexp = reinterpret_cast<int32_t*>(p);
    p += 256;
    int32_t* dexp = reinterpret_cast<int32_t*>(p);
    p += round_up(((size_t)cand_per_pass + 1) * 4, 256);
    uint16_t* xt = reinterpret_cast<uint16_t*>(p);
    p += round_up((size_t)d_in * (size_t)awq::gram_n_pad(n_tokens) * 2, 256);
    float* g32 = reinterpret_cast<float*>(p);
    uint16_t* d16 = static_cast<uint16_t*>(delta);
    e = awq::launch_gram(x, ld_x, n_tokens, d_in, xt, g32, g16, gexp, st);
    if (e != hipSuccess) return hip_fail(e, "gram launch");
    for (int k0 = 0; k0 < n_grid; k0 += cand_per_pass) {
      const int nk = n_grid - k0 < cand_per_pass ? n_grid - k0 : cand_per_pass;
      const double* cs = cand_scales + (int64_t)k0 * d_in;
      double* ts = tile_sse + (int64_t)k0 * tiles;
      if ((e = awq::launch_delta_exp(w, d_in, cs, nk, bound_b, dexp, st)) != hipSuccess)
        return hip_fail(e, "delta_exp launch");
      e = quantizer == AWQ_QUANT_INT4_GROUP ? awq::launch_quant_delta_f16(w, d_in, cs, nk, d16, dexp, st)
                                            : awq::launch_quant_delta_row_f16(w, d_in, quantizer, cs, nk, d16, dexp, st);
      if (e != hipSuccess) return hip_fail(e, "quant_delta_f16 launch");
      if ((e = awq::launch_fill_f64(ts, (int64_t)nk * tiles, 0.0, st)) != hipSuccess) return hip_fail(e, "fill launch");
      if ((e = awq::launch_quad_sse(g16, gexp, d16, dexp, nk, d_in, d_out, tiles, ts, st)) != hipSuccess)
        return hip_fail(e, "gram_error_sse launch");
    }
    e = awq::launch_loss_argmin(tile_sse, tiles, n_grid, n_tokens, d_out, cand_scales, d_in, losses,
                                best_scales, best_info, st);
    if (e != hipSuccess) return hip_fail(e, "loss_argmin launch");
    return ok();
  }
  for (int k0 = 0; k0 < n_grid; k0 += cand_per_pass) {
    const int nk = n_grid - k0 < cand_per_pass ? n_grid - k0 : cand_per_pass;
    const double* cs = cand_scales + (int64_t)k0 * d_in;
    e = quantizer == AWQ_QUANT_INT4_GROUP ? awq::launch_quant_delta(w, dtype, d_in, cs, nk, delta, st)
                                          : awq::launch_quant_delta_row(w, dtype, d_in, quantizer, cs, nk, delta, st);
    if (e != hipSuccess) return hip_fail(e, "quant_delta launch");
    e = awq::launch_error_sse(x, ld_x, delta, dtype, n_tokens, d_in, d_out, nk, tile_sse + (int64_t)k0 * tiles, st);
    if (e != hipSuccess) return hip_fail(e, "error_sse launch");
  }
  e = awq::launch_loss_argmin(tile_sse, tiles, n_grid, n_tokens, d_out, cand_scales, d_in, losses,
                              best_scales, best_info, st);
  if (e != hipSuccess) return hip_fail(e, "loss_argmin launch");
  return ok();
}

int check_mlp_dims(int64_t n_tokens, int64_t d_in, int64_t d_ff) {
  if (n_tokens < 0) return fail(AWQ_ERR_SHAPE, "n_tokens %lld < 0", (long long)n_tokens);
  if (n_tokens == 0) return fail(AWQ_ERR_NO_TOKENS, "n_tokens == 0");
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  if (d_ff <= 0 || d_ff % AWQ_GROUP_SIZE)
    return fail(AWQ_ERR_SHAPE, "d_ff %lld is not a positive multiple of 128", (long long)d_ff);
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_in));
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_ff));
  if (n_tokens > ((int64_t)1 << 40) / d_ff) return fail(AWQ_ERR_UNSUPPORTED, "n_tokens * d_ff too large");
  return AWQ_OK;
}

}  // namespace

extern "C" {

int awq_abi_version(void) { return AWQ_ABI_VERSION; }

const char* awq_status_string(int status) {
  switch (status) {
    case AWQ_OK: return "AWQ_OK";
    case AWQ_ERR_NULL: return "AWQ_ERR_NULL";
    case AWQ_ERR_SHAPE: return "AWQ_ERR_SHAPE";
    case AWQ_ERR_NO_TOKENS: return "AWQ_ERR_NO_TOKENS";
    case AWQ_ERR_ARG: return "AWQ_ERR_ARG";
    case AWQ_ERR_UNSUPPORTED: return "AWQ_ERR_UNSUPPORTED";
    case AWQ_ERR_WORKSPACE: return "AWQ_ERR_WORKSPACE";
    case AWQ_ERR_HIP: return "AWQ_ERR_HIP";
    default: return "AWQ_STATUS_UNKNOWN";
  }
}

const char* awq_last_error(void) { return g_err; }

size_t awq_act_stats_workspace_bytes(int dtype, int64_t n_tokens, int64_t d_in) {
  if ((dtype != AWQ_DTYPE_BF16 && dtype != AWQ_DTYPE_F32) || n_tokens <= 0 || d_in <= 0 ||
      d_in % AWQ_GROUP_SIZE)
    return 0;
  const awq::ActStatsPlan p = awq::act_stats_plan(dtype, n_tokens, d_in);
  return round_up((size_t)p.row_chunks * (size_t)d_in * sizeof(double), 256);
}

int awq_act_stats(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                  double* act_mean, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_x(x, dtype, n_tokens, d_in, ld_x));
  if (!act_mean) return fail(AWQ_ERR_NULL, "act_mean is NULL");
  const size_t need = awq_act_stats_workspace_bytes(dtype, n_tokens, d_in);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  const awq::ActStatsPlan p = awq::act_stats_plan(dtype, n_tokens, d_in);
  hipError_t e = awq::launch_act_stats(x, dtype, n_tokens, d_in, ld_x, act_mean,
                                       static_cast<double*>(workspace), p, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "act_stats launch");
  return ok();
}

int awq_candidate_scales(const double* act_mean, int64_t d_in, int n_grid, double* cand_scales,
                         void* stream) {
  if (!act_mean || !cand_scales) return fail(AWQ_ERR_NULL, "act_mean or cand_scales is NULL");
  if (d_in <= 0) return fail(AWQ_ERR_SHAPE, "d_in %lld must be > 0", (long long)d_in);
  if (n_grid < 1 || n_grid > 65535) return fail(AWQ_ERR_ARG, "n_grid %d outside [1, 65535]", n_grid);
  hipError_t e = awq::launch_candidate_scales(act_mean, d_in, n_grid, cand_scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "candidate_scales launch");
  return ok();
}

int awq_quant_delta(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                    int64_t d_in, int group_size, const double* cand_scales, int n_cand,
                    void* delta, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(group_size, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  if (!cand_scales || !delta) return fail(AWQ_ERR_NULL, "cand_scales or delta is NULL");
  if (n_cand < 1) return fail(AWQ_ERR_ARG, "n_cand %d < 1", n_cand);
  if (!aligned(delta, 16)) return fail(AWQ_ERR_UNSUPPORTED, "delta is not 16-byte aligned");
  // the kernel reads the scales two float64 at a time
  if (!aligned(cand_scales, 16)) return fail(AWQ_ERR_UNSUPPORTED, "cand_scales is not 16-byte aligned");
  hipError_t e = awq::launch_quant_delta(w, dtype, d_in, cand_scales, n_cand, delta, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quant_delta launch");
  return ok();
}

int64_t awq_error_tiles(int64_t n_tokens, int64_t d_out) {
  if (n_tokens <= 0 || d_out <= 0) return 0;
  return ((n_tokens + awq::kTileM - 1) / awq::kTileM) * ((d_out + awq::kTileN - 1) / awq::kTileN);
}

int awq_error_sse(const void* x, int64_t ld_x, const void* delta, int dtype, int64_t n_tokens,
                  int64_t d_in, int64_t d_out, int n_cand, double* tile_sse, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  TRY(check_x(x, dtype, n_tokens, d_in, ld_x));
  if (!delta || !tile_sse) return fail(AWQ_ERR_NULL, "delta or tile_sse is NULL");
  if (!aligned(delta, 16)) return fail(AWQ_ERR_UNSUPPORTED, "delta is not 16-byte aligned");
  if (d_out <= 0) return fail(AWQ_ERR_SHAPE, "d_out %lld must be > 0", (long long)d_out);
  if (n_cand < 1) return fail(AWQ_ERR_ARG, "n_cand %d < 1", n_cand);
  const int64_t blocks = awq_error_tiles(n_tokens, d_out) * n_cand;
  if (blocks > 0x7FFFFFFF) return fail(AWQ_ERR_UNSUPPORTED, "%lld tiles exceed one launch", (long long)blocks);
  hipError_t e = awq::launch_error_sse(x, ld_x, delta, dtype, n_tokens, d_in, d_out, n_cand, tile_sse,
                                       (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "error_sse launch");
  return ok();
}

int awq_loss_argmin(const double* tile_sse, int64_t tiles_per_cand, int n_grid, int64_t n_tokens,
                    int64_t d_out, const double* cand_scales, int64_t d_in, double* losses,
                    double* best_scales, int32_t* best_info, void* stream) {
  if (!tile_sse || !cand_scales || !losses || !best_scales || !best_info)
    return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (tiles_per_cand <= 0 || n_tokens <= 0 || d_out <= 0 || d_in <= 0)
    return fail(AWQ_ERR_SHAPE, "sizes must be > 0");
  if (n_grid < 1 || n_grid > 65535) return fail(AWQ_ERR_ARG, "n_grid %d outside [1, 65535]", n_grid);
  hipError_t e = awq::launch_loss_argmin(tile_sse, tiles_per_cand, n_grid, n_tokens, d_out, cand_scales,
                                         d_in, losses, best_scales, best_info, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "loss_argmin launch");
  return ok();
}

size_t awq_search_workspace_bytes(int dtype, int64_t n_tokens, int64_t d_in, int64_t d_out,
                                  int group_size, int n_grid, int cand_per_pass) {
  if ((dtype != AWQ_DTYPE_BF16 && dtype != AWQ_DTYPE_F32) || n_tokens <= 0 || d_in <= 0 || d_out <= 0 ||
      group_size != AWQ_GROUP_SIZE || d_in % group_size || n_grid < 1 || cand_per_pass < 1 ||
      cand_per_pass > n_grid)
    return 0;
  const size_t delta = round_up((size_t)cand_per_pass * (size_t)d_out * (size_t)d_in * esize(dtype), 256);
  const size_t sse = round_up((size_t)n_grid * (size_t)awq_error_tiles(n_tokens, d_out) * sizeof(double), 256);
  const size_t gram = gram_form(dtype, n_tokens, d_in, d_out, n_grid) ? gram_search_extra(n_tokens, d_in, cand_per_pass) : 0;
  return delta + sse + gram;
}

int awq_search_loss_form(int dtype, int64_t n_tokens, int64_t d_in, int64_t d_out, int n_grid) {
  return gram_form(dtype, n_tokens, d_in, d_out, n_grid) ? AWQ_LOSS_GRAM : AWQ_LOSS_DIRECT;
}

size_t awq_gram_workspace_bytes(int64_t n_tokens, int64_t d_in) {
  if (n_tokens <= 0 || d_in <= 0 || d_in % AWQ_GROUP_SIZE) return 0;
  return gram_ws_bytes(n_tokens, d_in);
}

int awq_gram(const void* x, int64_t ld_x, int64_t n_tokens, int64_t d_in, uint16_t* gram, int32_t* gram_exp,
             void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_in));
  TRY(check_x(x, AWQ_DTYPE_BF16, n_tokens, d_in, ld_x));
  if (!gram || !gram_exp) return fail(AWQ_ERR_NULL, "gram or gram_exp is NULL");
  if (!aligned(gram, 16) || !aligned(gram_exp, 4)) return fail(AWQ_ERR_UNSUPPORTED, "gram is not 16-byte aligned");
  if ((int64_t)awq::kTileM * awq::gram_n_pad(n_tokens) * 2 > 0x7FFFFFFF)
    return fail(AWQ_ERR_UNSUPPORTED, "n_tokens %lld too large for 32-bit tile offsets", (long long)n_tokens);
  const size_t need = gram_ws_bytes(n_tokens, d_in);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  uint16_t* xt = static_cast<uint16_t*>(workspace);
  float* g32 = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                        round_up((size_t)d_in * (size_t)awq::gram_n_pad(n_tokens) * 2, 256));
  hipError_t e = awq::launch_gram(x, ld_x, n_tokens, d_in, xt, g32, gram, gram_exp, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "gram launch");
  return ok();
}

int awq_quant_delta_f16(const void* const* w_parts, const int64_t* part_rows, int n_parts, int64_t d_in,
                        int group_size, const double* cand_scales, int n_cand, uint16_t* delta, int32_t* delta_exp,
                        void* stream) {
  TRY(check_group(group_size, d_in));
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_in));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, AWQ_DTYPE_BF16, d_in, &w));
  if (!cand_scales || !delta || !delta_exp) return fail(AWQ_ERR_NULL, "cand_scales, delta or delta_exp is NULL");
  if (n_cand < 1 || n_cand > 65535) return fail(AWQ_ERR_ARG, "n_cand %d outside [1, 65535]", n_cand);
  if (!aligned(delta, 16)) return fail(AWQ_ERR_UNSUPPORTED, "delta is not 16-byte aligned");
  if (!aligned(cand_scales, 16)) return fail(AWQ_ERR_UNSUPPORTED, "cand_scales is not 16-byte aligned");
  if (!aligned(delta_exp, 4)) return fail(AWQ_ERR_UNSUPPORTED, "delta_exp is not 4-byte aligned");
  hipError_t e = awq::launch_delta_exp(w, d_in, cand_scales, n_cand, 1e-8, delta_exp, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "delta_exp launch");
  e = awq::launch_quant_delta_f16(w, d_in, cand_scales, n_cand, delta, delta_exp, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quant_delta_f16 launch");
  return ok();
}

int awq_gram_error_sse(const uint16_t* gram, const int32_t* gram_exp, const uint16_t* delta,
                       const int32_t* delta_exp, int n_cand, int64_t n_tokens, int64_t d_in, int64_t d_out,
                       double* tile_sse, void* stream) {
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_in));
  if (!gram || !gram_exp || !delta || !delta_exp || !tile_sse) return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(gram, 16) || !aligned(delta, 16)) return fail(AWQ_ERR_UNSUPPORTED, "gram or delta is not 16-byte aligned");
  if (!aligned(gram_exp, 4) || !aligned(delta_exp, 4) || !aligned(tile_sse, 8))
    return fail(AWQ_ERR_UNSUPPORTED, "gram_exp, delta_exp or tile_sse is misaligned");
  if (d_out <= 0) return fail(AWQ_ERR_SHAPE, "d_out %lld must be > 0", (long long)d_out);
  if (n_tokens < d_in)
    return fail(AWQ_ERR_SHAPE, "n_tokens %lld < d_in %lld: the Gram form's tiles do not fit the loss layout",
                (long long)n_tokens, (long long)d_in);
  if (n_cand < 1 || n_cand > 65535) return fail(AWQ_ERR_ARG, "n_cand %d outside [1, 65535]", n_cand);
  if (d_out > ((int64_t)1 << 40) / d_in) return fail(AWQ_ERR_UNSUPPORTED, "d_out * d_in too large");
  const int64_t stride = awq_error_tiles(n_tokens, d_out);
  const int64_t blocks = ((d_in + awq::kTileM - 1) / awq::kTileM) * ((d_out + awq::kTileN - 1) / awq::kTileN) * n_cand;
  if (blocks > 0x7FFFFFFF || stride * n_cand > 0x7FFFFFFF)
    return fail(AWQ_ERR_UNSUPPORTED, "%lld tiles exceed one launch", (long long)blocks);
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = awq::launch_fill_f64(tile_sse, stride * n_cand, 0.0, st);
  if (e != hipSuccess) return hip_fail(e, "fill launch");
  e = awq::launch_quad_sse(gram, gram_exp, delta, delta_exp, n_cand, d_in, d_out, stride, tile_sse, st);
  if (e != hipSuccess) return hip_fail(e, "gram_error_sse launch");
  return ok();
}

int awq_search_scales(const void* x, int64_t ld_x, const void* const* w_parts,
                      const int64_t* part_rows, int n_parts, int dtype, int64_t n_tokens,
                      int64_t d_in, const double* act_mean, int group_size, int n_grid,
                      int cand_per_pass, double* cand_scales, double* losses,
                      double* best_scales, int32_t* best_info, void* workspace,
                      size_t workspace_bytes, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(group_size, d_in));
  return run_search(x, ld_x, w_parts, part_rows, n_parts, dtype, n_tokens, d_in, act_mean, nullptr, nullptr,
                    AWQ_FORMULA_MSMODELSLIM, AWQ_QUANT_INT4_GROUP, n_grid, cand_per_pass, cand_scales, losses,
                    best_scales, best_info, workspace, workspace_bytes, stream);
}

int awq_quantize_pack(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype,
                      int64_t d_in, int group_size, const double* s, uint8_t* codes,
                      float* qscales, int32_t* zeros, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(group_size, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  if (!s || !codes || !qscales || !zeros) return fail(AWQ_ERR_NULL, "s, codes, qscales or zeros is NULL");
  if (!aligned(codes, 16) || !aligned(qscales, 4) || !aligned(zeros, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "codes must be 16-byte aligned, qscales and zeros 4-byte aligned");
  // the kernel reads s two float64 at a time
  if (!aligned(s, 16)) return fail(AWQ_ERR_UNSUPPORTED, "s is not 16-byte aligned");
  hipError_t e = awq::launch_quantize_pack(w, dtype, d_in, s, codes, qscales, zeros, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quantize_pack launch");
  return ok();
}

int awq_act_stats_accumulate(const void* x, int dtype, int64_t n_tokens, int64_t d_in, int64_t ld_x,
                             double* sums, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_x(x, dtype, n_tokens, d_in, ld_x));
  if (!sums) return fail(AWQ_ERR_NULL, "sums is NULL");
  const size_t need = awq_act_stats_workspace_bytes(dtype, n_tokens, d_in);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  const awq::ActStatsPlan p = awq::act_stats_plan(dtype, n_tokens, d_in);
  hipError_t e = awq::launch_act_stats(x, dtype, n_tokens, d_in, ld_x, sums, static_cast<double*>(workspace), p,
                                       (hipStream_t)stream, true);
  if (e != hipSuccess) return hip_fail(e, "act_stats launch");
  return ok();
}

int awq_act_stats_finalize(const double* sums, int64_t d_in, int64_t total_tokens, double* act_mean,
                           void* stream) {
  if (!sums || !act_mean) return fail(AWQ_ERR_NULL, "sums or act_mean is NULL");
  if (d_in <= 0) return fail(AWQ_ERR_SHAPE, "d_in %lld must be > 0", (long long)d_in);
  if (total_tokens < 0) return fail(AWQ_ERR_SHAPE, "total_tokens %lld < 0", (long long)total_tokens);
  if (total_tokens == 0) return fail(AWQ_ERR_NO_TOKENS, "total_tokens is 0: no activation mean");
  hipError_t e = awq::launch_act_mean_from_sums(sums, d_in, total_tokens, act_mean, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "act_stats_finalize launch");
  return ok();
}

int awq_fold_scales(const void* src, int64_t ld_src, int dtype, int64_t rows, int64_t cols, const double* s,
                    void* dst, int64_t ld_dst, void* stream) {
  TRY(check_dtype(dtype));
  if (!src || !s || !dst) return fail(AWQ_ERR_NULL, "src, s or dst is NULL");
  if (rows <= 0 || cols <= 0) return fail(AWQ_ERR_SHAPE, "rows %lld and cols %lld must be > 0", (long long)rows,
                                          (long long)cols);
  if (ld_src < cols || ld_dst < cols)
    return fail(AWQ_ERR_ARG, "ld_src %lld / ld_dst %lld < cols %lld", (long long)ld_src, (long long)ld_dst,
                (long long)cols);
  const size_t es = esize(dtype);
  if (!aligned(src, es) || !aligned(dst, es)) return fail(AWQ_ERR_UNSUPPORTED, "src or dst is not element-aligned");
  if (cols > ((int64_t)1 << 31) - 256) return fail(AWQ_ERR_UNSUPPORTED, "cols %lld too large", (long long)cols);
  // 16-byte vectors when every row start is 16-byte aligned and the rows are whole vectors
  const bool vec = cols % 8 == 0 && aligned(src, 16) && aligned(dst, 16) && ld_src % (16 / (int64_t)es) == 0 &&
                   ld_dst % (16 / (int64_t)es) == 0;
  hipError_t e = awq::launch_fold_scales(src, ld_src, dtype, rows, cols, s, dst, ld_dst, vec, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fold_scales launch");
  return ok();
}

namespace {
int check_heads(int64_t n_heads, int64_t n_kv_heads, int64_t head_dim) {
  if (n_heads <= 0 || n_kv_heads <= 0 || head_dim <= 0)
    return fail(AWQ_ERR_SHAPE, "n_heads %lld, n_kv_heads %lld and head_dim %lld must be > 0", (long long)n_heads,
                (long long)n_kv_heads, (long long)head_dim);
  if (n_heads % n_kv_heads)
    return fail(AWQ_ERR_SHAPE, "n_heads %lld is not a multiple of n_kv_heads %lld", (long long)n_heads,
                (long long)n_kv_heads);
  if (n_heads > (1 << 20) || head_dim > (1 << 20) || n_heads * head_dim > ((int64_t)1 << 31))
    return fail(AWQ_ERR_UNSUPPORTED, "n_heads * head_dim too large");
  return AWQ_OK;
}
}  // namespace

int awq_tie_heads(const double* act_mean, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, double* tied,
                  void* stream) {
  if (!act_mean || !tied) return fail(AWQ_ERR_NULL, "act_mean or tied is NULL");
  TRY(check_heads(n_heads, n_kv_heads, head_dim));
  hipError_t e = awq::launch_tie_heads(act_mean, n_heads, n_kv_heads, head_dim, tied, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "tie_heads launch");
  return ok();
}

int awq_head_group_scales(const double* s, int64_t n_heads, int64_t n_kv_heads, int64_t head_dim, double* s_kv,
                          void* stream) {
  if (!s || !s_kv) return fail(AWQ_ERR_NULL, "s or s_kv is NULL");
  TRY(check_heads(n_heads, n_kv_heads, head_dim));
  hipError_t e = awq::launch_head_group_scales(s, n_heads, n_kv_heads, head_dim, s_kv, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "head_group_scales launch");
  return ok();
}

int awq_export_fp16(const float* qscales, const int32_t* zeros, int64_t rows, int64_t n_groups, uint16_t* steps_f16,
                    uint8_t* zeros_u4, int32_t* counts, void* stream) {
  if (!qscales || !zeros || !steps_f16 || !zeros_u4 || !counts)
    return fail(AWQ_ERR_NULL, "qscales, zeros, steps_f16, zeros_u4 or counts is NULL");
  if (rows <= 0 || n_groups <= 0)
    return fail(AWQ_ERR_SHAPE, "rows %lld and n_groups %lld must be > 0", (long long)rows, (long long)n_groups);
  if (rows > ((int64_t)1 << 40) / ((n_groups + 1) / 2)) return fail(AWQ_ERR_UNSUPPORTED, "export too large");
  if (!aligned(qscales, 4) || !aligned(zeros, 4) || !aligned(steps_f16, 2) || !aligned(counts, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "qscales, zeros, counts must be 4-byte and steps_f16 2-byte aligned");
  hipError_t e = awq::launch_export_fp16(qscales, zeros, rows, n_groups, steps_f16, zeros_u4, counts,
                                         (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "export_fp16 launch");
  return ok();
}

int awq_weight_mean(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype, int64_t d_in,
                    double* w_mean, void* workspace, size_t workspace_bytes, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  if (!w_mean) return fail(AWQ_ERR_NULL, "w_mean is NULL");
  size_t need = 0;
  for (int p = 0; p < n_parts; ++p) {
    const size_t b = awq_act_stats_workspace_bytes(dtype, part_rows[p], d_in);
    need = b > need ? b : need;
  }
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  // column sums of |W| part by part (the statistic's kernels, W's rows in place of tokens), then
  // one division by the stacked row count
  hipError_t e = awq::launch_fill(w_mean, d_in, 0.0, st);
  if (e != hipSuccess) return hip_fail(e, "weight_mean fill");
  for (int p = 0; p < n_parts; ++p) {
    const awq::ActStatsPlan plan = awq::act_stats_plan(dtype, part_rows[p], d_in);
    e = awq::launch_act_stats(w_parts[p], dtype, part_rows[p], d_in, d_in, w_mean, static_cast<double*>(workspace),
                              plan, st, true);
    if (e != hipSuccess) return hip_fail(e, "weight_mean column sums");
  }
  e = awq::launch_act_mean_from_sums(w_mean, d_in, w.row_begin[w.n], w_mean, st);
  if (e != hipSuccess) return hip_fail(e, "weight_mean division");
  return ok();
}

int awq_candidate_scales_ex(const double* act_mean, const double* w_mean, int64_t d_in, const double* ratios,
                            int n_ratios, int formula, double* cand_scales, void* stream) {
  if (!act_mean || !cand_scales) return fail(AWQ_ERR_NULL, "act_mean or cand_scales is NULL");
  if (d_in <= 0) return fail(AWQ_ERR_SHAPE, "d_in %lld must be > 0", (long long)d_in);
  awq::RatioList rl;
  TRY(check_ratios(ratios, n_ratios, formula, w_mean, &rl));
  hipError_t e = awq::launch_candidate_scales_ex(act_mean, w_mean, d_in, rl, n_ratios, formula, cand_scales,
                                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "candidate_scales_ex launch");
  return ok();
}

int awq_quant_delta_ex(const void* const* w_parts, const int64_t* part_rows, int n_parts, int dtype, int64_t d_in,
                       int quantizer, const double* cand_scales, int n_cand, void* delta, void* stream) {
  TRY(check_quantizer(quantizer));
  if (quantizer == AWQ_QUANT_INT4_GROUP)
    return awq_quant_delta(w_parts, part_rows, n_parts, dtype, d_in, AWQ_GROUP_SIZE, cand_scales, n_cand, delta,
                           stream);
  TRY(check_dtype(dtype));
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  if (!cand_scales || !delta) return fail(AWQ_ERR_NULL, "cand_scales or delta is NULL");
  if (n_cand < 1) return fail(AWQ_ERR_ARG, "n_cand %d < 1", n_cand);
  if (!aligned(delta, 16) || !aligned(cand_scales, 16))
    return fail(AWQ_ERR_UNSUPPORTED, "delta and cand_scales must be 16-byte aligned");
  hipError_t e = awq::launch_quant_delta_row(w, dtype, d_in, quantizer, cand_scales, n_cand, delta,
                                             (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "quant_delta_ex launch");
  return ok();
}

int awq_search_scales_ex(const void* x, int64_t ld_x, const void* const* w_parts, const int64_t* part_rows,
                         int n_parts, int dtype, int64_t n_tokens, int64_t d_in, const double* act_mean,
                         const double* w_mean, const double* ratios, int n_ratios, int formula, int quantizer,
                         int cand_per_pass, double* cand_scales, double* losses, double* best_scales,
                         int32_t* best_info, void* workspace, size_t workspace_bytes, void* stream) {
  if (!ratios) return fail(AWQ_ERR_NULL, "ratios is NULL");
  return run_search(x, ld_x, w_parts, part_rows, n_parts, dtype, n_tokens, d_in, act_mean, w_mean, ratios, formula,
                    quantizer, n_ratios, cand_per_pass, cand_scales, losses, best_scales, best_info, workspace,
                    workspace_bytes, stream);
}

int awq_w4a16_gemm(const void* x, int64_t ld_x, int x_dtype, const uint8_t* codes, const uint16_t* steps_f16,
                   const uint8_t* zeros_u4, int64_t n_tokens, int64_t d_in, int64_t d_out, void* y, int64_t ld_y,
                   int y_dtype, void* stream) {
  if (x_dtype != AWQ_DTYPE_BF16 && x_dtype != AWQ_DTYPE_F16)
    return fail(AWQ_ERR_UNSUPPORTED, "x_dtype %d: the activations are AWQ_DTYPE_BF16 or AWQ_DTYPE_F16", x_dtype);
  if (y_dtype != AWQ_DTYPE_F32 && y_dtype != x_dtype)
    return fail(AWQ_ERR_UNSUPPORTED, "y_dtype %d: AWQ_DTYPE_F32 or x_dtype", y_dtype);
  if (n_tokens < 0 || d_out <= 0)
    return fail(AWQ_ERR_SHAPE, "n_tokens %lld must be >= 0 and d_out %lld > 0", (long long)n_tokens,
                (long long)d_out);
  if (n_tokens == 0) return fail(AWQ_ERR_NO_TOKENS, "n_tokens == 0");
  TRY(check_group(AWQ_GROUP_SIZE, d_in));
  if (!x || !codes || !steps_f16 || !zeros_u4 || !y) return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (ld_x < d_in) return fail(AWQ_ERR_ARG, "ld_x %lld < d_in %lld", (long long)ld_x, (long long)d_in);
  if (ld_y < d_out) return fail(AWQ_ERR_ARG, "ld_y %lld < d_out %lld", (long long)ld_y, (long long)d_out);
  if (ld_x % 8 || !aligned(x, 16)) return fail(AWQ_ERR_UNSUPPORTED, "x must be 16-byte aligned with ld_x % 8 == 0");
  if (!aligned(codes, 16) || !aligned(steps_f16, 2))
    return fail(AWQ_ERR_UNSUPPORTED, "codes must be 16-byte and steps_f16 2-byte aligned");
  if (!aligned(y, y_dtype == AWQ_DTYPE_F32 ? 4 : 2)) return fail(AWQ_ERR_UNSUPPORTED, "y is not element-aligned");
  if (n_tokens > 0x7FFFFFFF - 256 || d_out > 0x7FFFFFFF - 256)
    return fail(AWQ_ERR_UNSUPPORTED, "sizes beyond the kernels' 32-bit indices");
  // the many-token kernel's activation offsets (128 tokens of ld_x) and per-wave code ranges (64
  // rows of d_in / 2 bytes) are 32-bit: the GEMMs' 256-row tile bound covers both
  TRY(check_d_in_bytes(AWQ_DTYPE_BF16, d_in));
  if (ld_x > kMaxTileBytes || (int64_t)awq::kTileM * ld_x * 2 > kMaxTileBytes)
    return fail(AWQ_ERR_UNSUPPORTED, "ld_x %lld too large for 32-bit tile offsets", (long long)ld_x);
  hipError_t e = awq::launch_w4a16_gemm(x, ld_x, x_dtype == AWQ_DTYPE_F16 ? 1 : 0, codes, steps_f16, zeros_u4,
                                        n_tokens, d_in, d_out, y, ld_y, y_dtype == AWQ_DTYPE_F32,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "w4a16_gemm launch");
  return ok();
}

int awq_mlp_hidden_ref(const void* x, int64_t ld_x, const void* w_gate, const void* w_up, int64_t n_tokens,
                       int64_t d_in, int64_t d_ff, float* g_ref, float* u_ref, void* stream) {
  TRY(check_mlp_dims(n_tokens, d_in, d_ff));
  TRY(check_x(x, AWQ_DTYPE_BF16, n_tokens, d_in, ld_x));
  if (!w_gate || !w_up || !g_ref || !u_ref) return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(g_ref, 4) || !aligned(u_ref, 4))
    return fail(AWQ_ERR_UNSUPPORTED, "w_gate / w_up must be 16-byte and g_ref / u_ref 4-byte aligned");
  hipError_t e = awq::launch_mlp_hidden(awq::kModeRef, awq::kActSilu, x, ld_x, w_gate, w_up, n_tokens, d_in, d_ff,
                                        g_ref, u_ref, nullptr, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mlp_hidden_ref launch");
  return ok();
}

int awq_mlp_hidden_delta(const void* x, int64_t ld_x, const void* dw_gate, const void* dw_up, const float* g_ref,
                         const float* u_ref, int act, int64_t n_tokens, int64_t d_in, int64_t d_ff, void* dh,
                         void* stream) {
  if (act != AWQ_ACT_SILU && act != AWQ_ACT_RELU) return fail(AWQ_ERR_ARG, "act %d is not an awq_act", act);
  TRY(check_mlp_dims(n_tokens, d_in, d_ff));
  TRY(check_x(x, AWQ_DTYPE_BF16, n_tokens, d_in, ld_x));
  if (!dw_gate || !dw_up || !g_ref || !u_ref || !dh) return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(dw_gate, 16) || !aligned(dw_up, 16) || !aligned(g_ref, 4) || !aligned(u_ref, 4) || !aligned(dh, 2))
    return fail(AWQ_ERR_UNSUPPORTED, "dw_gate / dw_up must be 16-byte, g_ref / u_ref 4-byte, dh 2-byte aligned");
  hipError_t e = awq::launch_mlp_hidden(awq::kModeDelta, act, x, ld_x, dw_gate, dw_up, n_tokens, d_in, d_ff,
                                        const_cast<float*>(g_ref), const_cast<float*>(u_ref), dh,
                                        (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "mlp_hidden_delta launch");
  return ok();
}

size_t awq_search_workspace_bytes_mlp(int64_t n_tokens, int64_t d_in, int64_t d_ff, int64_t d_model, int n_grid,
                                      int cand_per_pass) {
  if (n_tokens <= 0 || d_in <= 0 || d_in % AWQ_GROUP_SIZE || d_ff <= 0 || d_ff % AWQ_GROUP_SIZE || d_model <= 0 ||
      n_grid < 1 || cand_per_pass < 1 || cand_per_pass > n_grid)
    return 0;
  const size_t delta = round_up((size_t)cand_per_pass * 2 * (size_t)d_ff * (size_t)d_in * 2, 256);
  const size_t gu = 2 * round_up((size_t)n_tokens * (size_t)d_ff * 4, 256);
  const size_t dh = round_up((size_t)n_tokens * (size_t)d_ff * 2, 256);
  const size_t sse = round_up((size_t)n_grid * (size_t)awq_error_tiles(n_tokens, d_model) * sizeof(double), 256);
  return delta + gu + dh + sse;
}

int awq_search_scales_mlp(const void* x, int64_t ld_x, const void* w_gate, const void* w_up, const void* w_down,
                          int64_t n_tokens, int64_t d_in, int64_t d_ff, int64_t d_model, const double* act_mean,
                          int act, int n_grid, int cand_per_pass, double* cand_scales, double* losses,
                          double* best_scales, int32_t* best_info, void* workspace, size_t workspace_bytes,
                          void* stream) {
  if (act != AWQ_ACT_SILU && act != AWQ_ACT_RELU) return fail(AWQ_ERR_ARG, "act %d is not an awq_act", act);
  TRY(check_mlp_dims(n_tokens, d_in, d_ff));
  TRY(check_x(x, AWQ_DTYPE_BF16, n_tokens, d_in, ld_x));
  if (d_model <= 0) return fail(AWQ_ERR_SHAPE, "d_model %lld must be > 0", (long long)d_model);
  if (!w_gate || !w_up || !w_down || !act_mean || !cand_scales || !losses || !best_scales || !best_info)
    return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(w_gate, 16) || !aligned(w_up, 16) || !aligned(w_down, 16))
    return fail(AWQ_ERR_UNSUPPORTED, "weights must be 16-byte aligned");
  if (!aligned(cand_scales, 16)) return fail(AWQ_ERR_UNSUPPORTED, "cand_scales is not 16-byte aligned");
  if (d_ff > ((int64_t)65535 * 128) / 2) return fail(AWQ_ERR_UNSUPPORTED, "d_ff %lld too large", (long long)d_ff);
  if (n_grid < 1 || n_grid > 65535) return fail(AWQ_ERR_ARG, "n_grid %d outside [1, 65535]", n_grid);
  if (cand_per_pass < 1 || cand_per_pass > n_grid)
    return fail(AWQ_ERR_ARG, "cand_per_pass %d outside [1, n_grid]", cand_per_pass);
  const size_t need = awq_search_workspace_bytes_mlp(n_tokens, d_in, d_ff, d_model, n_grid, cand_per_pass);
  if (!workspace || workspace_bytes < need)
    return fail(AWQ_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace ? workspace_bytes : 0, need);
  if (!aligned(workspace, 256)) return fail(AWQ_ERR_UNSUPPORTED, "workspace is not 256-byte aligned");

  hipStream_t st = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  uint16_t* delta = reinterpret_cast<uint16_t*>(ws);
  ws += round_up((size_t)cand_per_pass * 2 * (size_t)d_ff * (size_t)d_in * 2, 256);
  float* g_ref = reinterpret_cast<float*>(ws);
  ws += round_up((size_t)n_tokens * (size_t)d_ff * 4, 256);
  float* u_ref = reinterpret_cast<float*>(ws);
  ws += round_up((size_t)n_tokens * (size_t)d_ff * 4, 256);
  uint16_t* dh = reinterpret_cast<uint16_t*>(ws);
  ws += round_up((size_t)n_tokens * (size_t)d_ff * 2, 256);
  double* tile_sse = reinterpret_cast<double*>(ws);
  const int64_t tiles = awq_error_tiles(n_tokens, d_model);

  const void* parts[2] = {w_gate, w_up};
  const int64_t rows[2] = {d_ff, d_ff};
  awq::WParts w;
  TRY(make_parts(parts, rows, 2, AWQ_DTYPE_BF16, d_in, &w));

  hipError_t e = awq::launch_candidate_scales(act_mean, d_in, n_grid, cand_scales, st);
  if (e != hipSuccess) return hip_fail(e, "candidate_scales launch");
  e = awq::launch_mlp_hidden(awq::kModeRef, act, x, ld_x, w_gate, w_up, n_tokens, d_in, d_ff, g_ref, u_ref, nullptr,
                             st);
  if (e != hipSuccess) return hip_fail(e, "mlp_hidden_ref launch");
  for (int k0 = 0; k0 < n_grid; k0 += cand_per_pass) {
    const int nk = n_grid - k0 < cand_per_pass ? n_grid - k0 : cand_per_pass;
    e = awq::launch_quant_delta(w, AWQ_DTYPE_BF16, d_in, cand_scales + (int64_t)k0 * d_in, nk, delta, st);
    if (e != hipSuccess) return hip_fail(e, "quant_delta launch");
    for (int k = 0; k < nk; ++k) {
      const uint16_t* dwg = delta + (int64_t)k * 2 * d_ff * d_in;
      e = awq::launch_mlp_hidden(awq::kModeDelta, act, x, ld_x, dwg, dwg + d_ff * d_in, n_tokens, d_in, d_ff, g_ref,
                                 u_ref, dh, st);
      if (e != hipSuccess) return hip_fail(e, "mlp_hidden_delta launch");
      e = awq::launch_error_sse(dh, d_ff, w_down, AWQ_DTYPE_BF16, n_tokens, d_ff, d_model, 1,
                                tile_sse + (int64_t)(k0 + k) * tiles, st);
      if (e != hipSuccess) return hip_fail(e, "error_sse launch");
    }
  }
  e = awq::launch_loss_argmin(tile_sse, tiles, n_grid, n_tokens, d_model, cand_scales, d_in, losses, best_scales,
                              best_info, st);
  if (e != hipSuccess) return hip_fail(e, "loss_argmin launch");
  return ok();
}

}  // extern "C"

// ------------------------------------------------------------------ search without allocation

namespace {

// Device scratch of awq_search_scales_noalloc: the tile sums of every candidate, then the delta of
// one candidate for one chunk of whole 256-row tiles. Every call on a GPU uses that GPU's copy of
// this array (held from the library's first use on the device until the process ends), so calls
// that overlap on one GPU race. In host code `scratch` stands for the device variable and is not a
// device address: its address comes from hipGetSymbolAddress, per device.
constexpr size_t kNoAllocScratchBytes = AWQ_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// This device's address of `scratch`, looked up once per device (with that device current).
int scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(AWQ_ERR_UNSUPPORTED, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || !aligned(p, 256)) return fail(AWQ_ERR_HIP, "scratch has no usable device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return AWQ_OK;
}

// Stacked rows [r0, r1) of a fused set, as a set of parts of their own.
awq::WParts slice_rows(const awq::WParts& w, int64_t r0, int64_t r1, int64_t row_bytes) {
  awq::WParts out;
  memset(&out, 0, sizeof out);
  int n = 0;
  for (int p = 0; p < w.n; ++p) {
    const int64_t b = w.row_begin[p], e = w.row_begin[p + 1];
    const int64_t lo = b > r0 ? b : r0, hi = e < r1 ? e : r1;
    if (lo >= hi) continue;
    out.ptr[n] = static_cast<const char*>(w.ptr[p]) + (lo - b) * row_bytes;
    out.row_begin[n] = lo - r0;
    ++n;
  }
  out.n = n;
  for (int p = n; p <= awq::kMaxParts; ++p) out.row_begin[p] = r1 - r0;
  return out;
}

}  // namespace

extern "C" {

int awq_search_scales_noalloc(const void* x, int64_t ld_x, const void* const* w_parts, const int64_t* part_rows,
                              int n_parts, int dtype, int64_t n_tokens, int64_t d_in, const double* act_mean,
                              int group_size, int n_grid, double* cand_scales, double* losses, double* best_scales,
                              int32_t* best_info, void* stream) {
  TRY(check_dtype(dtype));
  TRY(check_group(group_size, d_in));
  TRY(check_d_in_bytes(dtype, d_in));
  TRY(check_x(x, dtype, n_tokens, d_in, ld_x));
  awq::WParts w;
  TRY(make_parts(w_parts, part_rows, n_parts, dtype, d_in, &w));
  const int64_t d_out = w.row_begin[w.n];
  if (!act_mean || !cand_scales || !losses || !best_scales || !best_info)
    return fail(AWQ_ERR_NULL, "a required pointer is NULL");
  if (!aligned(cand_scales, 16)) return fail(AWQ_ERR_UNSUPPORTED, "cand_scales is not 16-byte aligned");
  if (n_grid < 1 || n_grid > 65535) return fail(AWQ_ERR_ARG, "n_grid %d outside [1, 65535]", n_grid);
  // scratch plan: tile sums of all candidates, then the delta of the largest chunk of whole
  // 256-row tiles (all rows when they fit) that the rest of the scratch holds
  const int64_t tiles_m = (n_tokens + awq::kTileM - 1) / awq::kTileM;
  const int64_t tiles = awq_error_tiles(n_tokens, d_out);
  const size_t sse_bytes = round_up((size_t)n_grid * (size_t)tiles * sizeof(double), 256);
  const size_t row_bytes = (size_t)d_in * esize(dtype);
  if (sse_bytes >= kNoAllocScratchBytes)
    return fail(AWQ_ERR_WORKSPACE, "%d candidates x %lld tiles of sums exceed the %zu-byte scratch", n_grid,
                (long long)tiles, kNoAllocScratchBytes);
  const int64_t fit_rows = (int64_t)((kNoAllocScratchBytes - sse_bytes) / row_bytes);
  const int64_t chunk = d_out <= fit_rows ? d_out : fit_rows / awq::kTileN * awq::kTileN;
  if (chunk < 1)
    return fail(AWQ_ERR_WORKSPACE, "the %zu-byte scratch holds no 256-row chunk of delta (d_in %lld)",
                kNoAllocScratchBytes, (long long)d_in);
  void* base = nullptr;
  TRY(scratch_on_current_device(&base));
  double* tile_sse = static_cast<double*>(base);
  void* delta = static_cast<char*>(base) + sse_bytes;

  hipStream_t st = (hipStream_t)stream;
  hipError_t e = awq::launch_candidate_scales(act_mean, d_in, n_grid, cand_scales, st);
  if (e != hipSuccess) return hip_fail(e, "candidate_scales launch");
  // the tile sums of candidate k are laid out as the one-launch search lays them out per candidate
  // (tiles_m x tiles_n, here chunk after chunk: token tile major within each chunk), and the
  // loss is their fixed-order sum as there; every value is written before it is read, so nothing
  // needs clearing
  for (int64_t r0 = 0; r0 < d_out; r0 += chunk) {
    const int64_t r1 = r0 + chunk < d_out ? r0 + chunk : d_out;
    const awq::WParts wc = slice_rows(w, r0, r1, (int64_t)row_bytes);
    for (int k = 0; k < n_grid; ++k) {
      e = awq::launch_quant_delta(wc, dtype, d_in, cand_scales + (int64_t)k * d_in, 1, delta, st);
      if (e != hipSuccess) return hip_fail(e, "quant_delta launch");
      e = awq::launch_error_sse(x, ld_x, delta, dtype, n_tokens, d_in, r1 - r0, 1,
                                tile_sse + (int64_t)k * tiles + tiles_m * (r0 / awq::kTileN), st);
      if (e != hipSuccess) return hip_fail(e, "error_sse launch");
    }
  }
  e = awq::launch_loss_argmin(tile_sse, tiles, n_grid, n_tokens, d_out, cand_scales, d_in, losses, best_scales,
                              best_info, st);
  if (e != hipSuccess) return hip_fail(e, "loss_argmin launch");
  return ok();
}

}  // extern "C"
