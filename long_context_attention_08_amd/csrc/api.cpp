// C ABI of libdsv4attn: argument validation (host only, before any HIP call),
// dispatch to the launchers, status strings.  See include/dsv4attn.h.
#include "../../include/dsv4attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <utility>

#include "dsv4_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return DSV4_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(DSV4_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool act_ok(int dt) { return dt == DSV4_F32 || dt == DSV4_BF16; }

// layouts usable for KV rows (compressed entries and window rows)
bool kv_layout_ok(int layout, int c) {
  if (layout == DSV4_ROW_F32 || layout == DSV4_ROW_BF16) return c >= 1;
  if (layout == DSV4_ROW_FP8_ROPE_BF16) return c >= 64 && c % 16 == 0;
  return false;
}

int check_ptrs16(const char* fn, std::initializer_list<std::pair<const void*, const char*>> ps) {
  for (auto& p : ps) {
    if (!p.first) return fail(DSV4_ERR_INVALID_ARG, "%s: %s is NULL", fn, p.second);
    if (!aligned16(p.first)) return fail(DSV4_ERR_INVALID_ARG, "%s: %s is not 16-byte aligned", fn, p.second);
  }
  return DSV4_OK;
}

}  // namespace

extern "C" {

size_t dsv4_row_bytes(int layout, int c) {
  if (c <= 0) return 0;
  switch (layout) {
    case DSV4_ROW_F32: return (size_t)4 * c;
    case DSV4_ROW_BF16: return (size_t)2 * c;
    case DSV4_ROW_FP8_ROPE_BF16: return c >= 64 ? (size_t)c + 64 : 0;
    case DSV4_ROW_MXFP4: return c % 32 == 0 ? (size_t)c / 2 : 0;
    default: return 0;
  }
}

const char* dsv4_status_string(int status) {
  switch (status) {
    case DSV4_OK: return "ok";
    case DSV4_ERR_INVALID_ARG: return "invalid argument";
    case DSV4_ERR_UNSUPPORTED: return "unsupported dtype/layout/shape combination";
    case DSV4_ERR_HIP: return "HIP launch error";
    case DSV4_ERR_WORKSPACE: return "workspace too small";
    default: return "unknown status";
  }
}

const char* dsv4_last_error(void) { return g_err; }

// --------------------------------------------------------------------------- compressors

static int check_csa_extra(const char* fn, int64_t n_left, int64_t n, int m, int64_t block0);
static int check_compress(const char* fn, const void* H, int64_t n_left, int64_t n, int64_t d, int act,
                          const void* W, const float* bias, int m, int c, void* comp, void* scales,
                          int comp_layout, void* raw, int raw_layout) {
  if (n_left < 0 || n < 0 || d <= 0 || c <= 0 || m <= 0)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes (n_left=%lld n=%lld d=%lld m=%d c=%d)", fn,
                (long long)n_left, (long long)n, (long long)d, m, c);
  if (!act_ok(act)) return fail(DSV4_ERR_UNSUPPORTED, "%s: act_dtype %d", fn, act);
  if (comp_layout == DSV4_ROW_MXFP4) {
    if (c % 32) return fail(DSV4_ERR_UNSUPPORTED, "%s: MXFP4 output needs c %% 32 == 0 (c=%d)", fn, c);
  } else if (!kv_layout_ok(comp_layout, c)) {
    return fail(DSV4_ERR_UNSUPPORTED, "%s: comp_layout %d with c=%d", fn, comp_layout, c);
  }
  if (raw && !kv_layout_ok(raw_layout, c)) return fail(DSV4_ERR_UNSUPPORTED, "%s: raw_layout %d with c=%d", fn, raw_layout, c);
  if (n_left + n == 0) return DSV4_OK;
  int r = check_ptrs16(fn, {{H, "H"}, {W, "W"}});
  if (r) return r;
  if (!bias) return fail(DSV4_ERR_INVALID_ARG, "%s: bias is NULL", fn);
  if (n / m > 0) {
    r = check_ptrs16(fn, {{comp, "comp_out"}});
    if (r) return r;
    if (comp_layout == DSV4_ROW_MXFP4 && !scales) return fail(DSV4_ERR_INVALID_ARG, "%s: comp_scales is NULL", fn);
  }
  if (raw && !aligned16(raw)) return fail(DSV4_ERR_INVALID_ARG, "%s: raw_out is not 16-byte aligned", fn);
  if (act == DSV4_BF16 && d % 8) return fail(DSV4_ERR_UNSUPPORTED, "%s: bf16 needs d %% 8 == 0", fn);
  return DSV4_OK;
}

int dsv4_csa_compress(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype,
                      const void* W, const float* bias_ab, int m, int c, int64_t block0,
                      void* comp_out, void* comp_scales, int comp_layout,
                      void* raw_out, int raw_layout, void* stream) {
  const char* fn = "dsv4_csa_compress";
  int r = check_compress(fn, H, n_left, n, d, act_dtype, W, bias_ab, m, c, comp_out, comp_scales,
                         comp_layout, raw_out, raw_layout);
  if (r) return r;
  r = check_csa_extra(fn, n_left, n, m, block0);
  if (r) return r;
  if (n == 0) return ok();
  dsv4::CompressArgs a{H, n_left, n, d, act_dtype, W, bias_ab, m, c, block0, comp_out,
                       reinterpret_cast<uint8_t*>(comp_scales), comp_layout, raw_out, raw_layout};
  return hip_status(dsv4::launch_csa_compress(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_hca_compress(const void* H, int64_t n, int64_t d, int act_dtype,
                      const void* W, const float* bias, int m_prime, int c,
                      void* comp_out, void* comp_scales, int comp_layout,
                      void* raw_out, int raw_layout, void* stream) {
  const char* fn = "dsv4_hca_compress";
  int r = check_compress(fn, H, 0, n, d, act_dtype, W, bias, m_prime, c, comp_out, comp_scales,
                         comp_layout, raw_out, raw_layout);
  if (r) return r;
  if (n == 0) return ok();
  dsv4::CompressArgs a{H, 0, n, d, act_dtype, W, bias, m_prime, c, 0, comp_out,
                       reinterpret_cast<uint8_t*>(comp_scales), comp_layout, raw_out, raw_layout};
  return hip_status(dsv4::launch_hca_compress(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

static int check_csa_extra(const char* fn, int64_t n_left, int64_t n, int m, int64_t block0) {
  if (m > 64) return fail(DSV4_ERR_UNSUPPORTED, "%s: m=%d > 64", fn, m);
  if (block0 < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: block0 < 0", fn);
  if (block0 >= 1 && n >= m && n_left < m)
    return fail(DSV4_ERR_INVALID_ARG, "%s: entry %lld needs %d rows of left context, got n_left=%lld", fn,
                (long long)block0, m, (long long)n_left);
  return 0;
}

static int chunk_launch(const char* fn, const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                        int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                        int m_prime, const dsv4_compressor_t* hca, void* stream);

static int chunk_check(const char* fn, const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                       int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                       int m_prime, const dsv4_compressor_t* hca) {
  for (const dsv4_compressor_t* j : {csa_kv, csa_keys}) {
    if (!j) continue;
    int r = check_compress(fn, H, n_left, n, d, act_dtype, j->W, j->bias, m, j->c, j->comp_out, j->comp_scales,
                           j->comp_layout, j->raw_out, j->raw_layout);
    if (!r) r = check_csa_extra(fn, n_left, n, m, block0);
    if (r) return r;
  }
  if (hca) {
    int r = check_compress(fn, H, 0, n, d, act_dtype, hca->W, hca->bias, m_prime, hca->c, hca->comp_out,
                           hca->comp_scales, hca->comp_layout, hca->raw_out, hca->raw_layout);
    if (r) return r;
  }
  return DSV4_OK;
}

static int rope_args_ok(const char* fn, int c, float eps, float theta, int rope_dims);

// fp32 rows of the normalised compressors in the workspace: CSA KV entries,
// CSA KV window rows, HCA entries, HCA window rows (256-byte aligned each)
struct ChunkNrLayout {
  size_t o_kv, o_kvraw, o_hc, o_hcraw, bytes;
};
static ChunkNrLayout chunk_nr_layout(int64_t n, int m, int c_kv, int m_prime, int c_hca) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  ChunkNrLayout L{};
  size_t o = 0;
  L.o_kv = o; o = al(o + (c_kv > 0 && m > 0 ? (size_t)(n / m) * c_kv * 4 : 0));
  L.o_kvraw = o; o = al(o + (c_kv > 0 ? (size_t)n * c_kv * 4 : 0));
  L.o_hc = o; o = al(o + (c_hca > 0 && m_prime > 0 ? (size_t)(n / m_prime) * c_hca * 4 : 0));
  L.o_hcraw = o; o = al(o + (c_hca > 0 ? (size_t)n * c_hca * 4 : 0));
  L.bytes = o;
  return L;
}

size_t dsv4_compress_chunk_nr_workspace_size(int64_t n, int m, int c_kv, int m_prime, int c_hca) {
  if (n <= 0 || c_kv < 0 || c_hca < 0) return 0;
  return chunk_nr_layout(n, m, c_kv, m_prime, c_hca).bytes;
}

int dsv4_compress_chunk_nr(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                           int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                           int m_prime, const dsv4_compressor_t* hca, const dsv4_norm_rope_t* kv_nr,
                           const dsv4_norm_rope_t* hca_nr, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_compress_chunk_nr";
  int r = chunk_check(fn, H, n_left, n, d, act_dtype, m, block0, csa_kv, csa_keys, m_prime, hca);
  if (r) return r;
  // only a given compressor with its norm-rope descriptor is normalised
  const dsv4_norm_rope_t* kvn = csa_kv ? kv_nr : nullptr;
  const dsv4_norm_rope_t* hcn = hca ? hca_nr : nullptr;
  for (auto jn : {std::make_pair(csa_kv, kvn), std::make_pair(hca, hcn)}) {
    const dsv4_compressor_t* j = jn.first;
    const dsv4_norm_rope_t* nr = jn.second;
    if (!nr) continue;
    if (nr->norm != 0 && nr->norm != 1) return fail(DSV4_ERR_INVALID_ARG, "%s: norm must be 0 or 1", fn);
    if ((r = rope_args_ok(fn, j->c, nr->eps, nr->theta, nr->rope_dims))) return r;
    for (int lay : {j->comp_layout, j->raw_out ? j->raw_layout : DSV4_ROW_F32})
      if (lay != DSV4_ROW_F32 && lay != DSV4_ROW_BF16 && lay != DSV4_ROW_FP8_ROPE_BF16)
        return fail(DSV4_ERR_UNSUPPORTED, "%s: normalised rows in layout %d (F32, BF16 or FP8_ROPE_BF16)", fn, lay);
  }
  const ChunkNrLayout lay = chunk_nr_layout(n, m, kvn ? csa_kv->c : 0, m_prime, hcn ? hca->c : 0);
  if (ws_bytes < lay.bytes || (lay.bytes && !ws))
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, lay.bytes);
  if (lay.bytes && !aligned16(ws)) return fail(DSV4_ERR_INVALID_ARG, "%s: ws is not 16-byte aligned", fn);
  if (n == 0 || (!csa_kv && !csa_keys && !hca)) return ok();
  // the KV compressors write fp32 rows into the workspace; the indexer keys
  // are not normalised and go straight to their outputs
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  dsv4_compressor_t kv32{}, hc32{};
  if (csa_kv) kv32 = *csa_kv;
  if (hca) hc32 = *hca;
  if (kvn) {
    kv32.comp_out = w + lay.o_kv; kv32.comp_scales = nullptr; kv32.comp_layout = DSV4_ROW_F32;
    kv32.raw_out = csa_kv->raw_out ? w + lay.o_kvraw : nullptr; kv32.raw_layout = DSV4_ROW_F32;
  }
  if (hcn) {
    hc32.comp_out = w + lay.o_hc; hc32.comp_scales = nullptr; hc32.comp_layout = DSV4_ROW_F32;
    hc32.raw_out = hca->raw_out ? w + lay.o_hcraw : nullptr; hc32.raw_layout = DSV4_ROW_F32;
  }
  r = chunk_launch(fn, H, n_left, n, d, act_dtype, m, block0, csa_kv ? &kv32 : nullptr, csa_keys, m_prime,
                   hca ? &hc32 : nullptr, stream);
  if (r) return r;
  // RMSNorm + RoPE + packing at the rows' positions: chunk token i sits at
  // position m block0 + i; CSA entry s (absolute) at m (s + 1) - 1; HCA entry
  // i of the chunk at m block0 + m' (i + 1) - 1
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const int64_t p_tok = (int64_t)m * block0;
  auto prep = [&](const dsv4_norm_rope_t* nr, const void* in, void* out, int out_layout, int64_t rows, int c,
                  int64_t pos0, int64_t stride) {
    if (rows <= 0) return DSV4_OK;
    dsv4::KvPrepArgs a{in, DSV4_ROW_F32, out, out_layout, 1, rows, c, nr->norm ? nr->gamma : nullptr,
                       nr->norm ? nr->eps : 0.f, nr->theta, nr->rope_dims, stride, nr->norm};
    return hip_status(dsv4::launch_kv_prep(a, &pos0, s), fn);
  };
  if (kvn) {
    if ((r = prep(kvn, kv32.comp_out, csa_kv->comp_out, csa_kv->comp_layout, n / m, csa_kv->c,
                  (int64_t)m * (block0 + 1) - 1, m)))
      return r;
    if (csa_kv->raw_out &&
        (r = prep(kvn, kv32.raw_out, csa_kv->raw_out, csa_kv->raw_layout, n, csa_kv->c, p_tok, 1)))
      return r;
  }
  if (hcn) {
    if ((r = prep(hcn, hc32.comp_out, hca->comp_out, hca->comp_layout, n / m_prime, hca->c, p_tok + m_prime - 1,
                  m_prime)))
      return r;
    if (hca->raw_out && (r = prep(hcn, hc32.raw_out, hca->raw_out, hca->raw_layout, n, hca->c, p_tok, 1))) return r;
  }
  return ok();
}

int dsv4_compress_chunk(const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                        int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                        int m_prime, const dsv4_compressor_t* hca, void* stream) {
  const char* fn = "dsv4_compress_chunk";
  for (const dsv4_compressor_t* j : {csa_kv, csa_keys}) {
    if (!j) continue;
    int r = check_compress(fn, H, n_left, n, d, act_dtype, j->W, j->bias, m, j->c, j->comp_out, j->comp_scales,
                           j->comp_layout, j->raw_out, j->raw_layout);
    if (!r) r = check_csa_extra(fn, n_left, n, m, block0);
    if (r) return r;
  }
  if (hca) {
    int r = check_compress(fn, H, 0, n, d, act_dtype, hca->W, hca->bias, m_prime, hca->c, hca->comp_out,
                           hca->comp_scales, hca->comp_layout, hca->raw_out, hca->raw_layout);
    if (r) return r;
  }
  if (n == 0 || (!csa_kv && !csa_keys && !hca)) return ok();
  return chunk_launch(fn, H, n_left, n, d, act_dtype, m, block0, csa_kv, csa_keys, m_prime, hca, stream);
}

// the compressors of a validated chunk: one fused launch when every one can
// take it, else one launch each
static int chunk_launch(const char* fn, const void* H, int64_t n_left, int64_t n, int64_t d, int act_dtype, int m,
                        int64_t block0, const dsv4_compressor_t* csa_kv, const dsv4_compressor_t* csa_keys,
                        int m_prime, const dsv4_compressor_t* hca, void* stream) {
  const size_t esz = act_dtype == DSV4_F32 ? 4 : 2;
  const void* Hh = reinterpret_cast<const uint8_t*>(H) + (size_t)n_left * (size_t)d * esz;
  auto csa = [&](const dsv4_compressor_t* j) {
    return dsv4::CompressArgs{H, n_left, n, d, act_dtype, j->W, j->bias, m, j->c, block0, j->comp_out,
                              reinterpret_cast<uint8_t*>(j->comp_scales), j->comp_layout, j->raw_out, j->raw_layout};
  };
  dsv4::CompressArgs akv{}, aki{}, ahc{};
  if (csa_kv) akv = csa(csa_kv);
  if (csa_keys) aki = csa(csa_keys);
  if (hca)
    ahc = dsv4::CompressArgs{Hh, 0, n, d, act_dtype, hca->W, hca->bias, m_prime, hca->c, 0, hca->comp_out,
                             reinterpret_cast<uint8_t*>(hca->comp_scales), hca->comp_layout, hca->raw_out,
                             hca->raw_layout};
  const dsv4::CompressArgs *pkv = csa_kv ? &akv : nullptr, *pki = csa_keys ? &aki : nullptr,
                           *phc = hca ? &ahc : nullptr;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (dsv4::compress_fused_ok(pkv, pki, phc)) return hip_status(dsv4::launch_compress_fused(pkv, pki, phc, s), fn);
  for (const dsv4::CompressArgs* a : {pkv, pki}) {
    if (!a) continue;
    int r = hip_status(dsv4::launch_csa_compress(*a, s), fn);
    if (r) return r;
  }
  return phc ? hip_status(dsv4::launch_hca_compress(*phc, s), fn) : ok();
}

// --------------------------------------------------------------------------- indexer

int dsv4_indexer_score(const void* qI, int q_dtype, const float* wI,
                       const void* keys, const uint8_t* k_scales, int k_layout,
                       int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                       const int64_t* q_pos0, float* scores, void* stream) {
  const char* fn = "dsv4_indexer_score";
  if (B < 0 || nq < 0 || S < 0 || hI <= 0 || cI <= 0 || m <= 0)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!act_ok(q_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: q_dtype %d", fn, q_dtype);
  if (k_layout != DSV4_ROW_F32 && k_layout != DSV4_ROW_BF16 && k_layout != DSV4_ROW_MXFP4)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: k_layout %d", fn, k_layout);
  if (k_layout == DSV4_ROW_MXFP4 && cI % 32) return fail(DSV4_ERR_UNSUPPORTED, "%s: MXFP4 keys need cI %% 32 == 0", fn);
  if (B == 0 || nq == 0 || S == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  for (int64_t b = 0; b < B; ++b)
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
  int r = check_ptrs16(fn, {{qI, "qI"}, {keys, "keys"}, {scores, "scores"}});
  if (r) return r;
  if (!wI) return fail(DSV4_ERR_INVALID_ARG, "%s: wI is NULL", fn);
  if (k_layout == DSV4_ROW_MXFP4 && !k_scales) return fail(DSV4_ERR_INVALID_ARG, "%s: k_scales is NULL", fn);
  dsv4::IndexerArgs a{qI, q_dtype, wI, keys, k_scales, k_layout, B, nq, hI, cI, S, m, scores, 0};
  return hip_status(dsv4::launch_indexer(a, q_pos0, reinterpret_cast<hipStream_t>(stream)), fn);
}

static dsv4::IndexerArgs it_args(int q_dtype, int k_layout, int64_t B, int64_t nq, int hI, int cI, int64_t S, int m) {
  dsv4::IndexerArgs a{};
  a.q_dtype = q_dtype; a.k_layout = k_layout; a.B = B; a.nq = nq; a.hI = hI; a.cI = cI; a.S = S; a.m = m;
  return a;
}

size_t dsv4_indexer_topk_workspace_size(int q_dtype, int k_layout, int64_t B, int64_t nq, int hI, int cI,
                                        int64_t S, int k) {
  if (B <= 0 || nq <= 0 || S <= 0 || hI <= 0 || cI <= 0 || k <= 0) return 0;
  return dsv4::idxtopk_workspace(it_args(q_dtype, k_layout, B, nq, hI, cI, S, 1), k);
}

int dsv4_indexer_topk(const void* qI, int q_dtype, const float* wI,
                      const void* keys, const uint8_t* k_scales, int k_layout,
                      int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                      const int64_t* q_pos0, int k, int32_t* idx_out,
                      void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_indexer_topk";
  if (B < 0 || nq < 0 || S < 0 || hI <= 0 || cI <= 0 || m <= 0 || k <= 0)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (k > 4096) return fail(DSV4_ERR_UNSUPPORTED, "%s: k=%d > 4096", fn, k);
  if (!act_ok(q_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: q_dtype %d", fn, q_dtype);
  if (k_layout != DSV4_ROW_F32 && k_layout != DSV4_ROW_BF16 && k_layout != DSV4_ROW_MXFP4)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: k_layout %d", fn, k_layout);
  if (k_layout == DSV4_ROW_MXFP4 && cI % 32) return fail(DSV4_ERR_UNSUPPORTED, "%s: MXFP4 keys need cI %% 32 == 0", fn);
  if (S >= (int64_t)1 << 31) return fail(DSV4_ERR_UNSUPPORTED, "%s: S >= 2^31", fn);
  if (B == 0 || nq == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  for (int64_t b = 0; b < B; ++b)
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
  if (!idx_out) return fail(DSV4_ERR_INVALID_ARG, "%s: idx_out is NULL", fn);
  const dsv4::IndexerArgs sz = it_args(q_dtype, k_layout, B, nq, hI, cI, S > 0 ? S : 1, m);
  const int64_t rows = B * nq < dsv4::MAXB * nq ? B * nq : dsv4::MAXB * nq;
  if (!dsv4::topk_make_plan(rows, S > 0 ? S : 1, k).supported)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: S=%lld with k=%d", fn, (long long)S, k);
  if (S > 0) {
    int r = check_ptrs16(fn, {{qI, "qI"}, {keys, "keys"}});
    if (r) return r;
    if (!wI) return fail(DSV4_ERR_INVALID_ARG, "%s: wI is NULL", fn);
    if (k_layout == DSV4_ROW_MXFP4 && !k_scales) return fail(DSV4_ERR_INVALID_ARG, "%s: k_scales is NULL", fn);
  }
  const size_t need = S > 0 ? dsv4::idxtopk_workspace(sz, k) : 0;
  if (ws_bytes < need || (need && !ws))
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, need);
  if (need && !aligned16(ws)) return fail(DSV4_ERR_INVALID_ARG, "%s: ws is not 16-byte aligned", fn);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (S == 0) {
    // nothing is visible: the top-k pass writes padding rows without reading scores
    const dsv4::TopkPlan tp = dsv4::topk_make_plan(rows, 1, k);
    return hip_status(dsv4::launch_topk(nullptr, B, nq, 0, m, q_pos0, k, idx_out, nullptr, tp, s), fn);
  }
  dsv4::IndexerArgs a = it_args(q_dtype, k_layout, B, nq, hI, cI, S, m);
  a.qI = qI; a.wI = wI; a.keys = keys; a.k_scales = k_scales;
  return hip_status(dsv4::launch_indexer_topk(a, q_pos0, k, idx_out, ws, s), fn);
}

static int indexer_quantised(const char* fn, int qfmt, const void* qI, int q_dtype, const float* wI,
                             const uint8_t* k_codes, const uint8_t* k_scales, int64_t B, int64_t nq, int hI,
                             int cI, int64_t S, int m, const int64_t* q_pos0, float* scores, void* stream) {
  if (B < 0 || nq < 0 || S < 0 || hI <= 0 || cI <= 0 || m <= 0)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!act_ok(q_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: q_dtype %d", fn, q_dtype);
  if (cI % 32) return fail(DSV4_ERR_UNSUPPORTED, "%s: cI %% 32 != 0", fn);
  if (B == 0 || nq == 0 || S == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  for (int64_t b = 0; b < B; ++b)
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
  int r = check_ptrs16(fn, {{qI, "qI"}, {k_codes, "k_codes"}, {scores, "scores"}});
  if (r) return r;
  if (!wI) return fail(DSV4_ERR_INVALID_ARG, "%s: wI is NULL", fn);
  if (!k_scales) return fail(DSV4_ERR_INVALID_ARG, "%s: k_scales is NULL", fn);
  dsv4::IndexerArgs a{qI, q_dtype, wI, k_codes, k_scales, DSV4_ROW_MXFP4, B, nq, hI, cI, S, m, scores, qfmt};
  return hip_status(dsv4::launch_indexer(a, q_pos0, reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_indexer_score_fp4q(const void* qI, int q_dtype, const float* wI,
                            const uint8_t* k_codes, const uint8_t* k_scales,
                            int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                            const int64_t* q_pos0, float* scores, void* stream) {
  return indexer_quantised("dsv4_indexer_score_fp4q", 4, qI, q_dtype, wI, k_codes, k_scales, B, nq, hI, cI, S, m,
                           q_pos0, scores, stream);
}

int dsv4_indexer_score_fp8q(const void* qI, int q_dtype, const float* wI,
                            const uint8_t* k_codes, const uint8_t* k_scales,
                            int64_t B, int64_t nq, int hI, int cI, int64_t S, int m,
                            const int64_t* q_pos0, float* scores, void* stream) {
  return indexer_quantised("dsv4_indexer_score_fp8q", 8, qI, q_dtype, wI, k_codes, k_scales, B, nq, hI, cI, S, m,
                           q_pos0, scores, stream);
}

// --------------------------------------------------------------------------- top-k

size_t dsv4_topk_workspace_size(int64_t B, int64_t nq, int64_t S, int k) {
  if (B <= 0 || nq <= 0 || S <= 0 || k <= 0) return 0;
  return dsv4::topk_make_plan(B * nq < dsv4::MAXB * nq ? B * nq : dsv4::MAXB * nq, S, k).bytes;
}

static int topk_check(const char* fn, const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                      const int64_t* q_pos0, int k, int32_t* idx_out, dsv4::TopkPlan* plan) {
  if (B < 0 || nq < 0 || S < 0 || m <= 0 || k <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (k > 4096) return fail(DSV4_ERR_UNSUPPORTED, "%s: k=%d > 4096", fn, k);
  if (B == 0 || nq == 0) return DSV4_OK;
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  for (int64_t b = 0; b < B; ++b)
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
  if (!idx_out) return fail(DSV4_ERR_INVALID_ARG, "%s: idx_out is NULL", fn);
  if (S > 0 && !scores) return fail(DSV4_ERR_INVALID_ARG, "%s: scores is NULL", fn);
  if (S >= (int64_t)1 << 31) return fail(DSV4_ERR_UNSUPPORTED, "%s: S >= 2^31", fn);
  const int64_t rows = B * nq < dsv4::MAXB * nq ? B * nq : dsv4::MAXB * nq;
  *plan = dsv4::topk_make_plan(rows, S > 0 ? S : 1, k);
  if (!plan->supported) return fail(DSV4_ERR_UNSUPPORTED, "%s: S=%lld with k=%d", fn, (long long)S, k);
  return DSV4_OK;
}

int dsv4_topk_select(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                     const int64_t* q_pos0, int k, int32_t* idx_out,
                     void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_topk_select";
  dsv4::TopkPlan plan{};
  int r = topk_check(fn, scores, B, nq, S, m, q_pos0, k, idx_out, &plan);
  if (r) return r;
  if (B == 0 || nq == 0) return ok();
  if (ws_bytes < plan.bytes || (plan.bytes && !ws))
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, plan.bytes);
  return hip_status(dsv4::launch_topk(scores, B, nq, S, m, q_pos0, k, idx_out, ws, plan,
                                      reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_topk_select_noalloc(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                             const int64_t* q_pos0, int k, int32_t* idx_out, void* stream) {
  const char* fn = "dsv4_topk_select_noalloc";
  dsv4::TopkPlan plan{};
  int r = topk_check(fn, scores, B, nq, S, m, q_pos0, k, idx_out, &plan);
  if (r) return r;
  if (B == 0 || nq == 0) return ok();
  if (plan.bytes > dsv4::TOPK_SCRATCH_BYTES)
    return fail(DSV4_ERR_UNSUPPORTED,
                "%s: this shape needs %zu bytes of workspace, more than the %zu the allocation-free call holds "
                "(use dsv4_topk_select with a workspace)", fn, plan.bytes, dsv4::TOPK_SCRATCH_BYTES);
  void* ws = nullptr;
  if (plan.bytes > 0) {
    r = hip_status(dsv4::topk_scratch_ptr(&ws), fn);
    if (r) return r;
  }
  return hip_status(dsv4::launch_topk(scores, B, nq, S, m, q_pos0, k, idx_out, ws, plan,
                                      reinterpret_cast<hipStream_t>(stream)), fn);
}

// --------------------------------------------------------------------------- attention

size_t dsv4_attn_workspace_size(int dense, int64_t B, int64_t nq, int nh, int c, int64_t max_keys) {
  if (B <= 0 || nq <= 0 || nh <= 0 || c <= 0) return 0;
  return dsv4::attn_workspace_bound(B, nq, nh, c, max_keys, dense != 0);
}

int dsv4_attn_plan(int dense, int q_dtype, int kv_layout, int64_t B, int64_t nq, int nh, int c, int64_t S,
                   int k, int m_prime, int n_win, const int64_t* q_pos0, dsv4_attn_plan_t* plan) {
  const char* fn = "dsv4_attn_plan";
  if (!plan) return fail(DSV4_ERR_INVALID_ARG, "%s: plan is NULL", fn);
  if (B < 0 || nq < 0 || nh <= 0 || c <= 0 || S < 0 || n_win < 0 || k < 0 || (dense && m_prime <= 0))
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (c > 1024 || !act_ok(q_dtype) || !kv_layout_ok(kv_layout, c))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: dtype, layout or c", fn);
  if (B > 0 && nq > 0 && !q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  for (int64_t b = 0; b < B && nq > 0; ++b)
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
  dsv4::AttnArgs a{};
  a.q_dtype = q_dtype; a.B = B; a.nq = nq; a.nh = nh; a.c = c; a.kv_layout = kv_layout; a.S = S;
  a.k = dense ? 0 : k; a.ratio = dense ? m_prime : 1; a.n_win = n_win; a.scale = 1.f;
  const dsv4::AttnLaunchPlan lp =
      dsv4::attn_make_plan(a, dense != 0, B > 0 && nq > 0 ? dsv4::attn_group_slots(a, q_pos0, dense != 0) : 0);
  plan->path = lp.path;
  plan->queries_per_block = lp.pl.qpw;
  plan->splits = lp.pl.max_splits;
  plan->split_slots = lp.pl.max_splits > 1 ? lp.pl.chunk : 0;
  plan->workspace_bytes = B > 0 && nq > 0 ? lp.ws_bytes : 0;
  return ok();
}

static int rope_args_ok(const char* fn, int c, float eps, float theta, int rope_dims);

static int attn_common(const char* fn, bool dense, const void* q, int q_dtype, int64_t B, int64_t nq, int nh,
                       int c, const void* kv_comp, int kv_layout, int64_t S, const int32_t* idx, int k,
                       int ratio, const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                       const int64_t* q_pos0, const float* sink, float scale, void* out, void* ws,
                       size_t ws_bytes, void* stream, float rot_theta = 0.f, int rot_dims = 0) {
  if (B < 0 || nq < 0 || nh <= 0 || c <= 0 || S < 0 || W < 0 || n_win < 0 || k < 0)
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (dense && ratio <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: m_prime <= 0", fn);
  if (c > 1024) return fail(DSV4_ERR_UNSUPPORTED, "%s: c=%d > 1024", fn, c);
  if (!act_ok(q_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: q_dtype %d", fn, q_dtype);
  if (!kv_layout_ok(kv_layout, c)) return fail(DSV4_ERR_UNSUPPORTED, "%s: kv_layout %d with c=%d", fn, kv_layout, c);
  if (!std::isfinite(scale) || !(scale > 0.0f)) return fail(DSV4_ERR_INVALID_ARG, "%s: scale must be finite and > 0", fn);
  if (rot_dims != 0) {
    int r = rope_args_ok(fn, c, 0.f, rot_theta, rot_dims);
    if (r) return r;
  }
  if (B == 0 || nq == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  int r = check_ptrs16(fn, {{q, "q"}, {out, "out"}});
  if (r) return r;
  if ((S > 0 && (dense || k > 0)) && (r = check_ptrs16(fn, {{kv_comp, "kv_comp"}}))) return r;
  if (!dense && k > 0 && !idx) return fail(DSV4_ERR_INVALID_ARG, "%s: idx is NULL", fn);
  if (n_win > 0) {
    if ((r = check_ptrs16(fn, {{kv_win, "kv_win"}}))) return r;
    if (!win_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: win_pos0 is NULL", fn);
  }
  for (int64_t b = 0; b < B; ++b) {
    if (q_pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0[%lld] < 0", fn, (long long)b);
    if (q_pos0[b] + nq >= ((int64_t)1 << 31)) return fail(DSV4_ERR_UNSUPPORTED, "%s: positions >= 2^31", fn);
    if (n_win > 0) {
      const int64_t p_first = q_pos0[b], p_last = q_pos0[b] + nq - 1;
      const int64_t lo = p_first - n_win + 1 > 0 ? p_first - n_win + 1 : 0;
      if (lo < win_pos0[b] || p_last >= win_pos0[b] + W)
        return fail(DSV4_ERR_INVALID_ARG,
                    "%s: batch %lld: window positions [%lld, %lld] not covered by kv_win rows [%lld, %lld)", fn,
                    (long long)b, (long long)lo, (long long)p_last, (long long)win_pos0[b],
                    (long long)(win_pos0[b] + W));
    }
  }
  dsv4::AttnArgs a{q, q_dtype, B, nq, nh, c, kv_comp, kv_layout, S, dense ? nullptr : idx, dense ? 0 : k,
                   dense ? ratio : 1, kv_win, W, n_win, sink, scale, out, ws, ws_bytes, rot_theta, rot_dims};
  // one plan serves the check and the launch
  const dsv4::AttnLaunchPlan plan = dsv4::attn_make_plan(a, dense, dsv4::attn_group_slots(a, q_pos0, dense));
  if (ws_bytes < plan.ws_bytes || (plan.ws_bytes && !ws))
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes, plan.ws_bytes);
  return hip_status(dsv4::launch_attn(a, q_pos0, win_pos0, plan, reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_sparse_mqa_fwd(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                        const void* kv_comp, int kv_layout, int64_t S,
                        const int32_t* idx, int k,
                        const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                        const int64_t* q_pos0, const float* sink, float scale,
                        void* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_common("dsv4_sparse_mqa_fwd", false, q, q_dtype, B, nq, nh, c, kv_comp, kv_layout, S, idx, k, 1,
                     kv_win, W, win_pos0, n_win, q_pos0, sink, scale, out, ws, ws_bytes, stream);
}

int dsv4_hca_dense_fwd(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                       const void* kv_comp, int kv_layout, int64_t S, int m_prime,
                       const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                       const int64_t* q_pos0, const float* sink, float scale,
                       void* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_common("dsv4_hca_dense_fwd", true, q, q_dtype, B, nq, nh, c, kv_comp, kv_layout, S, nullptr, 0,
                     m_prime, kv_win, W, win_pos0, n_win, q_pos0, sink, scale, out, ws, ws_bytes, stream);
}

int dsv4_sparse_mqa_fwd_rope(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                             const void* kv_comp, int kv_layout, int64_t S,
                             const int32_t* idx, int k,
                             const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                             const int64_t* q_pos0, const float* sink, float scale,
                             float theta, int rope_dims,
                             void* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_common("dsv4_sparse_mqa_fwd_rope", false, q, q_dtype, B, nq, nh, c, kv_comp, kv_layout, S, idx, k, 1,
                     kv_win, W, win_pos0, n_win, q_pos0, sink, scale, out, ws, ws_bytes, stream, theta, rope_dims);
}

int dsv4_hca_dense_fwd_rope(const void* q, int q_dtype, int64_t B, int64_t nq, int nh, int c,
                            const void* kv_comp, int kv_layout, int64_t S, int m_prime,
                            const void* kv_win, int64_t W, const int64_t* win_pos0, int n_win,
                            const int64_t* q_pos0, const float* sink, float scale,
                            float theta, int rope_dims,
                            void* out, void* ws, size_t ws_bytes, void* stream) {
  return attn_common("dsv4_hca_dense_fwd_rope", true, q, q_dtype, B, nq, nh, c, kv_comp, kv_layout, S, nullptr, 0,
                     m_prime, kv_win, W, win_pos0, n_win, q_pos0, sink, scale, out, ws, ws_bytes, stream, theta,
                     rope_dims);
}

// --------------------------------------------------------------------------- Q/KV norm and RoPE

static int rope_args_ok(const char* fn, int c, float eps, float theta, int rope_dims) {
  if (c <= 0 || c % 8 || c > 4096) return fail(DSV4_ERR_UNSUPPORTED, "%s: c=%d (multiple of 8, <= 4096)", fn, c);
  if (rope_dims < 0 || rope_dims > c || rope_dims % 8 || rope_dims > 512)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: rope_dims=%d (multiple of 8, <= min(c, 512))", fn, rope_dims);
  if (!(eps >= 0.f) || !(theta > 0.f)) return fail(DSV4_ERR_INVALID_ARG, "%s: eps < 0 or theta <= 0", fn);
  return 0;
}

int dsv4_q_norm_rope(const void* q, int q_dtype, void* q_out, int64_t B, int64_t nq, int nh, int c,
                     const float* gamma, float eps, float theta, int rope_dims,
                     const int64_t* q_pos0, void* stream) {
  const char* fn = "dsv4_q_norm_rope";
  if (B < 0 || nq < 0 || nh <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!act_ok(q_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: q_dtype %d", fn, q_dtype);
  int r = rope_args_ok(fn, c, eps, theta, rope_dims);
  if (r) return r;
  if (B == 0 || nq == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  r = check_ptrs16(fn, {{q, "q"}, {q_out, "q_out"}});
  if (r) return r;
  dsv4::QPrepArgs a{q, q_out, q_dtype, B, nq, nh, c, gamma, eps, theta, rope_dims, 0};
  return hip_status(dsv4::launch_q_prep(a, q_pos0, reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_kv_norm_rope(const void* rows, int in_layout, int64_t B, int64_t n, int c,
                      const float* gamma, float eps, float theta, int rope_dims,
                      const int64_t* pos0, int64_t pos_stride,
                      void* rows_out, int out_layout, void* stream) {
  const char* fn = "dsv4_kv_norm_rope";
  if (B < 0 || n < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (in_layout != DSV4_ROW_F32 && in_layout != DSV4_ROW_BF16)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: in_layout %d", fn, in_layout);
  if (out_layout != DSV4_ROW_F32 && out_layout != DSV4_ROW_BF16 && out_layout != DSV4_ROW_FP8_ROPE_BF16)
    return fail(DSV4_ERR_UNSUPPORTED, "%s: out_layout %d", fn, out_layout);
  int r = rope_args_ok(fn, c, eps, theta, rope_dims);
  if (r) return r;
  if (out_layout == DSV4_ROW_FP8_ROPE_BF16 && (c < 64 || c % 16))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: FP8 rows need c >= 64, c %% 16 == 0", fn);
  if (B == 0 || n == 0) return ok();
  if (!pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: pos0 is NULL", fn);
  r = check_ptrs16(fn, {{rows, "rows"}, {rows_out, "rows_out"}});
  if (r) return r;
  if (rows == rows_out && dsv4_row_bytes(in_layout, c) != dsv4_row_bytes(out_layout, c))
    return fail(DSV4_ERR_INVALID_ARG, "%s: in place needs equal row sizes", fn);
  dsv4::KvPrepArgs a{rows, in_layout, rows_out, out_layout, B, n, c, gamma, eps, theta, rope_dims, pos_stride, 1};
  return hip_status(dsv4::launch_kv_prep(a, pos0, reinterpret_cast<hipStream_t>(stream)), fn);
}

int dsv4_out_rope(void* o, int o_dtype, int64_t B, int64_t nq, int nh, int c, float theta, int rope_dims,
                  const int64_t* q_pos0, void* stream) {
  const char* fn = "dsv4_out_rope";
  if (B < 0 || nq < 0 || nh <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (!act_ok(o_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: o_dtype %d", fn, o_dtype);
  int r = rope_args_ok(fn, c, 0.f, theta, rope_dims);
  if (r) return r;
  if (B == 0 || nq == 0 || rope_dims == 0) return ok();
  if (!q_pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: q_pos0 is NULL", fn);
  r = check_ptrs16(fn, {{o, "o"}});
  if (r) return r;
  dsv4::QPrepArgs a{o, o, o_dtype, B, nq, nh, c, nullptr, 0.f, theta, rope_dims, 1};
  return hip_status(dsv4::launch_q_prep(a, q_pos0, reinterpret_cast<hipStream_t>(stream)), fn);
}

// --------------------------------------------------------------------------- streaming cache maintenance

size_t dsv4_stream_state_bytes(int overlap, int m, int c) {
  if ((overlap != 0 && overlap != 1) || m < 1 || c < 1) return 0;
  return dsv4::stream_state_bytes(overlap, m, c);
}

int dsv4_stream_state_reset(void* state, int64_t B, int overlap, int m, int c, void* stream) {
  const char* fn = "dsv4_stream_state_reset";
  if (B < 0 || m < 1 || m > 1024 || c < 1 || (overlap != 0 && overlap != 1))
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (B == 0) return ok();
  int r = check_ptrs16(fn, {{state, "state"}});
  if (r) return r;
  return hip_status(dsv4::launch_stream_reset(state, B, overlap, m, c, reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t dsv4_stream_workspace_size(int64_t B, int64_t n_new, int64_t d, int overlap, int c) {
  if (B <= 0 || n_new <= 0 || d <= 0 || c <= 0 || (overlap != 0 && overlap != 1)) return 0;
  return dsv4::stream_ws_bytes(B * n_new, overlap, c, d);
}

int64_t dsv4_swa_ring_pos0(int64_t p_last, int64_t ring_w) {
  if (ring_w <= 0) return 0;
  const int64_t x = p_last - ring_w + 1;
  const int64_t q = x >= 0 ? x / ring_w : -((-x + ring_w - 1) / ring_w);   // floor division
  return q * ring_w;
}

int dsv4_stream_compress(const void* H, int64_t B, int64_t n_new, int64_t d, int act_dtype,
                         const void* W, const float* bias, int overlap, int m, int c,
                         const int64_t* pos0, const int64_t* emit_from, void* state,
                         void* cache, void* cache_scales, int cache_layout, int64_t S,
                         void* ring, int64_t ring_w, int ring_layout, const dsv4_norm_rope_t* nr,
                         void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_stream_compress";
  if (B < 0 || n_new < 0 || d < 1 || S < 0 || m < 1 || m > 1024 || (overlap != 0 && overlap != 1))
    return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (c < 2 || c > 512 || c % 2) return fail(DSV4_ERR_UNSUPPORTED, "%s: c=%d (even, <= 512)", fn, c);
  if (!act_ok(act_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: act_dtype %d", fn, act_dtype);
  if (act_dtype == DSV4_BF16 && d % 8) return fail(DSV4_ERR_UNSUPPORTED, "%s: bf16 needs d %% 8 == 0", fn);
  if (cache && !kv_layout_ok(cache_layout, c) && !(cache_layout == DSV4_ROW_MXFP4 && c % 32 == 0))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: cache_layout %d with c=%d", fn, cache_layout, c);
  if (ring && !kv_layout_ok(ring_layout, c))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: ring_layout %d with c=%d", fn, ring_layout, c);
  if (ring && ring_w < 1) return fail(DSV4_ERR_INVALID_ARG, "%s: ring_w < 1", fn);
  if (nr) {
    int r = rope_args_ok(fn, c, nr->eps, nr->theta, nr->rope_dims);
    if (r) return r;
  }
  if (B == 0 || n_new == 0) return ok();
  if (!pos0) return fail(DSV4_ERR_INVALID_ARG, "%s: pos0 is NULL", fn);
  for (int64_t b = 0; b < B; ++b)
    if (pos0[b] < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: pos0[%lld] < 0", fn, (long long)b);
  int r = check_ptrs16(fn, {{H, "H"}, {W, "W"}, {state, "state"}, {ws, "ws"}});
  if (r) return r;
  if (!bias) return fail(DSV4_ERR_INVALID_ARG, "%s: bias is NULL", fn);
  if (cache && cache_layout == DSV4_ROW_MXFP4 && !cache_scales)
    return fail(DSV4_ERR_INVALID_ARG, "%s: cache_scales is NULL", fn);
  const size_t need = dsv4::stream_ws_bytes(B * n_new, overlap, c, d);
  if (ws_bytes < need)
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes, need);
  dsv4::StreamArgs a{};
  a.H = H; a.act = act_dtype; a.d = d; a.W = W; a.bias = bias;
  a.nmat = overlap ? 4 : 2; a.c = c; a.m = m; a.overlap = overlap;
  a.B = B; a.n_new = n_new; a.part = reinterpret_cast<float*>(ws); a.state = state;
  a.cache = S > 0 ? cache : nullptr; a.cache_scales = reinterpret_cast<uint8_t*>(cache_scales);
  a.cache_layout = cache_layout; a.S = S;
  a.ring = ring; a.ring_w = ring_w; a.ring_layout = ring_layout;
  if (nr) {
    a.norm = nr->norm ? 1 : 0; a.gamma = nr->gamma; a.eps = nr->eps; a.theta = nr->theta; a.rope_dims = nr->rope_dims;
  }
  return hip_status(dsv4::launch_stream(a, pos0, emit_from, reinterpret_cast<hipStream_t>(stream)), fn);
}

// --------------------------------------------------------------------------- projections (GEMM)

static int gemm_check(const char* fn, const void* A, int64_t lda, const void* B, int64_t ldb, const void* C,
                      int64_t ldc, int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 0 || K <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (K % 64) return fail(DSV4_ERR_UNSUPPORTED, "%s: K=%lld (multiple of 64)", fn, (long long)K);
  if (lda < K || ldb < K || ldc < N) return fail(DSV4_ERR_INVALID_ARG, "%s: leading dimension too small", fn);
  if (lda % 8 || ldb % 8) return fail(DSV4_ERR_UNSUPPORTED, "%s: lda, ldb must be multiples of 8", fn);
  if (M == 0 || N == 0) return 0;
  return check_ptrs16(fn, {{A, "A"}, {B, "B"}, {C, "C"}});
}

int dsv4_gemm_bf16_nt(const void* A, int64_t lda, int64_t stride_a, const void* B, int64_t ldb, int64_t stride_b,
                      void* C, int c_dtype, int64_t ldc, int64_t stride_c, int64_t M, int64_t N, int64_t K,
                      int64_t batch, void* stream) {
  const char* fn = "dsv4_gemm_bf16_nt";
  if (!act_ok(c_dtype)) return fail(DSV4_ERR_UNSUPPORTED, "%s: c_dtype %d", fn, c_dtype);
  if (batch < 0) return fail(DSV4_ERR_INVALID_ARG, "%s: batch < 0", fn);
  int r = gemm_check(fn, A, lda, B, ldb, C, ldc, M, N, K);
  if (r) return r;
  if (M == 0 || N == 0 || batch == 0) return ok();
  if (batch > 1 && (stride_a % 8 || stride_b % 8))
    return fail(DSV4_ERR_UNSUPPORTED, "%s: batch strides of A and B must be multiples of 8", fn);
  dsv4::GemmArgs a{A, lda, stride_a, B, ldb, stride_b, C, ldc, stride_c, c_dtype == DSV4_F32 ? 1 : 0, M, N, K, batch};
  return hip_status(dsv4::launch_gemm(a, reinterpret_cast<hipStream_t>(stream)), fn);
}

size_t dsv4_query_proj_workspace_size(int64_t n, int d_c) {
  return n > 0 && d_c > 0 ? (size_t)n * d_c * 2 : 0;
}

int dsv4_query_proj(const void* h, int64_t n, int d, const void* W_DQ, int d_c,
                    const void* W_UQ, int nh, int c, const void* W_IUQ, int hI, int cI, const void* W_w,
                    void* q, void* qI, float* wI, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_query_proj";
  if (n < 0 || d <= 0 || d_c <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (n == 0) return ok();
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool need_cq = q || qI;
  int r;
  if (need_cq) {
    if (ws_bytes < dsv4_query_proj_workspace_size(n, d_c) || !ws)
      return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes,
                  dsv4_query_proj_workspace_size(n, d_c));
    if ((r = gemm_check(fn, h, d, W_DQ, d, ws, d_c, n, d_c, d))) return r;
    if (q && (nh <= 0 || c <= 0 || (r = gemm_check(fn, ws, d_c, W_UQ, d_c, q, (int64_t)nh * c, n, (int64_t)nh * c, d_c))))
      return r ? r : fail(DSV4_ERR_INVALID_ARG, "%s: nh, c", fn);
    if (qI && (hI <= 0 || cI <= 0 ||
               (r = gemm_check(fn, ws, d_c, W_IUQ, d_c, qI, (int64_t)hI * cI, n, (int64_t)hI * cI, d_c))))
      return r ? r : fail(DSV4_ERR_INVALID_ARG, "%s: hI, cI", fn);
  }
  if (wI && (hI <= 0 || (r = gemm_check(fn, h, d, W_w, d, wI, hI, n, hI, d))))
    return r ? r : fail(DSV4_ERR_INVALID_ARG, "%s: hI", fn);
  hipError_t e = hipSuccess;
  if (need_cq) {
    e = dsv4::launch_gemm({h, d, 0, W_DQ, d, 0, ws, d_c, 0, 0, n, d_c, d, 1}, s);
    if (e == hipSuccess && q)
      e = dsv4::launch_gemm({ws, d_c, 0, W_UQ, d_c, 0, q, (int64_t)nh * c, 0, 0, n, (int64_t)nh * c, d_c, 1}, s);
    if (e == hipSuccess && qI)
      e = dsv4::launch_gemm({ws, d_c, 0, W_IUQ, d_c, 0, qI, (int64_t)hI * cI, 0, 0, n, (int64_t)hI * cI, d_c, 1}, s);
  }
  if (e == hipSuccess && wI) e = dsv4::launch_gemm({h, d, 0, W_w, d, 0, wI, hI, 0, 1, n, hI, d, 1}, s);
  return hip_status(e, fn);
}

size_t dsv4_output_proj_workspace_size(int64_t n, int g, int d_g) {
  return n > 0 && g > 0 && d_g > 0 ? (size_t)n * g * d_g * 2 : 0;
}

int dsv4_output_proj(const void* o, int64_t n, int nh, int c, int g, int d_g, const void* W_O1,
                     const void* W_O2, int d, void* out, void* ws, size_t ws_bytes, void* stream) {
  const char* fn = "dsv4_output_proj";
  if (n < 0 || nh <= 0 || c <= 0 || g <= 0 || d_g <= 0 || d <= 0) return fail(DSV4_ERR_INVALID_ARG, "%s: bad sizes", fn);
  if (nh % g) return fail(DSV4_ERR_INVALID_ARG, "%s: nh %% g != 0", fn);
  if (n == 0) return ok();
  if (ws_bytes < dsv4_output_proj_workspace_size(n, g, d_g) || !ws)
    return fail(DSV4_ERR_WORKSPACE, "%s: workspace %zu bytes, need %zu", fn, ws_bytes,
                dsv4_output_proj_workspace_size(n, g, d_g));
  const int64_t kg = (int64_t)(nh / g) * c, zw = (int64_t)g * d_g;
  int r = gemm_check(fn, o, (int64_t)nh * c, W_O1, kg, ws, zw, n, d_g, kg);
  if (r) return r;
  if ((r = gemm_check(fn, ws, zw, W_O2, zw, out, d, n, d, zw))) return r;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = dsv4::launch_gemm({o, (int64_t)nh * c, kg, W_O1, kg, (int64_t)d_g * kg, ws, zw, d_g, 0, n, d_g, kg, g}, s);
  if (e == hipSuccess) e = dsv4::launch_gemm({ws, zw, 0, W_O2, zw, 0, out, d, 0, 0, n, d, zw, 1}, s);
  return hip_status(e, fn);
}

}  // extern "C"
