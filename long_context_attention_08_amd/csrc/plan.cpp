// Host-side planning of the top-k and attention launches: which kernel runs,
// how a row or a query group is split into parts, and how many workspace
// bytes the launch writes.  The C ABI's size queries, its argument checks and
// the launchers all call these functions, so a workspace the checks accept is
// exactly the one the kernels use.  No HIP calls (plain host code).
#include "dsv4_internal.h"

namespace dsv4 {

// ------------------------------------------------------------------ top-k

// histogram select for few long rows: parts of at least 8192 scores, at most 64
static bool hs_plan(int64_t rows, int64_t S, int k, int* part, int* nparts) {
  if (k > SK_KMAX || rows >= 512 || S <= 16384) return false;
  int64_t np = (512 + rows - 1) / rows;
  const int64_t by_len = S / 8192;
  if (np > by_len) np = by_len;
  if (np > 64) np = 64;
  if (np < 2) np = 2;
  const int64_t p = (S + np - 1) / np;
  *part = (int)p;
  *nparts = (int)((S + p - 1) / p);
  return true;
}

static void topk_parts(int64_t rows, int64_t S, int k, int* part, int* nparts) {
  if (k <= SK_KMAX) {
    // streaming: whole rows when there are enough of them, else up to 16
    // parts of at least 16384 scores so that some 512 blocks run
    int np = 1;
    if (rows < 512 && S > 16384) {
      np = (int)((512 + rows - 1) / rows);
      const int64_t by_len = S / 16384;
      if (np > by_len) np = (int)by_len;
      if (np > 16) np = 16;
      if (np < 1) np = 1;
    }
    int64_t p = (S + np - 1) / np;
    p = (p + 3) / 4 * 4;                       // parts start 16-byte aligned in aligned rows
    *part = (int)p;
    *nparts = (int)((S + p - 1) / p);
    return;
  }
  int p = k <= 1024 ? 32768 : 16384;
  if (rows < 256 && S > 16384 && k <= 1024) p = 16384;   // more blocks for few rows
  int fit = 4096;                                         // short rows: a smaller LDS stage
  while (fit < S && fit < p) fit <<= 1;
  p = fit < p ? fit : p;
  *part = p;
  *nparts = (int)((S + p - 1) / p);
}

TopkPlan topk_make_plan(int64_t rows, int64_t S, int k) {
  TopkPlan t = {};
  if (rows <= 0 || S <= 0 || k <= 0) {
    t.kind = TOPK_STREAM;
    t.part = 1;
    t.nparts = 1;
    t.supported = k >= 1 && k <= 4096;
    return t;
  }
  if (hs_plan(rows, S, k, &t.part, &t.nparts)) {
    t.kind = TOPK_HIST;
    t.supported = true;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    size_t o = 0;
    t.o_suf = o; o = al(o + (size_t)rows * t.nparts * HS_SUF * 4);
    t.o_meta = o; o = al(o + (size_t)rows * 16);   // per-row threshold bin and counts
    t.o_win = o; o = al(o + (size_t)rows * k * 8);
    t.o_cand = o; o = al(o + (size_t)rows * HS_CAP * 8);
    t.bytes = o;
    return t;
  }
  topk_parts(rows, S, k, &t.part, &t.nparts);
  t.kind = k <= SK_KMAX ? TOPK_STREAM : TOPK_STAGE;
  t.supported = k <= 4096 && (t.nparts == 1 || (int64_t)t.nparts * k <= TK_MAX_CAND);
  t.bytes = t.nparts > 1 ? (size_t)rows * t.nparts * k * sizeof(uint64_t) : 0;
  return t;
}

// ------------------------------------------------------------------ indexer

bool indexer_mfma_ok(const IndexerArgs& a) {
  return a.q_dtype == ACT_BF16 && a.hI == 32 && (a.cI == 32 || a.cI == 64 || a.cI == 128) &&
         a.S < ((int64_t)1 << 25) &&                 // 16 score rows fit a buffer range below 2^31 bytes
         (a.k_layout == ROW_BF16 || a.k_layout == ROW_MXFP4);
}

// Query blocks of 16 queries (8 for bf16 queries at cI = 128), or single
// queries below 16 per sequence; the key range of a block is split so that
// about 4096 (2048 for single queries) blocks run.
IndexerGrid indexer_grid(const IndexerArgs& a, int nb) {
  IndexerGrid g = {};
  const int64_t ntiles = (a.S + IDX_KT - 1) / IDX_KT;
  int64_t target;
  if (a.nq >= 16) {
    g.qb = 4 * (a.qfmt == 0 && a.cI == 128 ? 2 : 4);
    target = 4096;
  } else {
    g.qb = 1;
    target = 2048;
  }
  g.qblocks = (a.nq + g.qb - 1) / g.qb;
  const int64_t units = g.qblocks * nb;
  int64_t splits = units > 0 ? (target + units - 1) / units : 1;
  if (splits > ntiles) splits = ntiles;
  if (splits < 1) splits = 1;
  const int64_t tps = ntiles > 0 ? (ntiles + splits - 1) / splits : 1;
  g.tps = (int)tps;
  g.splits = (int)(ntiles > 0 ? (ntiles + tps - 1) / tps : 1);
  return g;
}

// ------------------------------------------------------------------ index scores + top-k

// Sample rank of the threshold: with one sample per 32 keys, the number of a
// row's top-k scores that land in the sample has mean k / 32; ks sits six
// standard deviations above it, so the threshold almost never cuts into the
// top k, and about 32 ks scores pass it.
static int it_sample_rank(int k) {
  const double mu = (double)k / IT_STRIDE;
  int ks = (int)(mu + 6.0 * __builtin_sqrt(mu)) + 2;
  return ks < 1 ? 1 : ks;
}

IdxTopkPlan idxtopk_make_plan(const IndexerArgs& a, int k) {
  IdxTopkPlan p = {};
  const int64_t rows = a.B * a.nq;
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  p.ks = it_sample_rank(k);
  p.Ss = a.S / IT_STRIDE;
  p.fused = a.qfmt == 0 && indexer_mfma_ok(a) && k <= SK_KMAX &&
            (int64_t)IT_STRIDE * p.ks * 8 / 5 <= IT_SELCAP &&   // expected candidates well inside a select block
            p.Ss >= 4 * (int64_t)p.ks && rows > 0;
  if (p.fused) {
    p.grid = indexer_grid(a, (int)a.B);
    // slots per (row, split): four times the select block's share, at least 256
    int64_t cap = (int64_t)4 * IT_SELCAP / p.grid.splits;
    cap = cap < 256 ? 256 : (cap > IT_SELCAP ? IT_SELCAP : cap);
    p.cap = (int)((cap + 63) / 64 * 64);
    p.tk_sample = topk_make_plan(rows, p.Ss, p.ks);
    p.o_sscore = o; o = al(o + (size_t)rows * p.Ss * 4);
    p.o_sidx = o; o = al(o + (size_t)rows * p.ks * 4);
    p.o_stk = o; o = al(o + p.tk_sample.bytes);
    p.o_lkey = o; o = al(o + (size_t)rows * 4);
    p.o_cand = o; o = al(o + (size_t)rows * p.grid.splits * p.cap * 8);
    p.o_cnt = o; o = al(o + (size_t)rows * p.grid.splits * 4);
    p.o_flags = o; o = al(o + (size_t)rows * 4);
  }
  if (p.fused) {
    // the full-score top-k sees only flagged rows (almost never any): one
    // streaming block per row, a single launch that leaves at once otherwise
    p.tk_full = TopkPlan{};
    p.tk_full.kind = TOPK_STREAM;
    p.tk_full.part = (int)((a.S + 3) / 4 * 4);
    p.tk_full.nparts = 1;
    p.tk_full.supported = true;
    p.tk_full.bytes = 0;
  } else {
    p.tk_full = topk_make_plan(rows, a.S, k);
  }
  p.o_scores = o; o = al(o + (size_t)rows * a.S * 4);
  p.o_ftk = o; o = al(o + p.tk_full.bytes);
  p.bytes = o;
  return p;
}

size_t idxtopk_workspace(const IndexerArgs& a, int k) {
  if (a.B <= 0 || a.nq <= 0 || a.S <= 0) return 0;
  IndexerArgs s = a;
  s.B = a.B < MAXB ? a.B : MAXB;
  size_t best = idxtopk_make_plan(s, k).bytes;
  if (a.B > MAXB && a.B % MAXB) {
    s.B = a.B % MAXB;
    const size_t t = idxtopk_make_plan(s, k).bytes;
    best = t > best ? t : best;
  }
  return best;
}

// ------------------------------------------------------------------ streaming compressors

// slices of d for the projection partials: about 256 blocks for one row group,
// slices of at least 256 (a multiple of 32)
void stream_split(int64_t NC, int64_t d, int* ks, int64_t* kslice) {
  const int64_t col_blocks = (NC + STREAM_SP_COLS - 1) / STREAM_SP_COLS;
  int64_t want = (256 + col_blocks - 1) / col_blocks;
  const int64_t most = d / 256 > 1 ? d / 256 : 1;
  if (want > most) want = most;
  if (want < 1) want = 1;
  int64_t sl = (d + want - 1) / want;
  sl = (sl + 31) / 32 * 32;
  *kslice = sl;
  *ks = (int)((d + sl - 1) / sl);
}

// state: [header][max | sum | weighted sum] x c of the current entry, and for
// CSA the same for the next entry's b-part
size_t stream_state_bytes(int overlap, int m, int c) {
  (void)m;
  const size_t acc = (size_t)(overlap ? 6 : 3) * (size_t)c * 4;
  return (STREAM_META_BYTES + acc + 255) / 256 * 256;
}

size_t stream_ws_bytes(int64_t rows, int overlap, int c, int64_t d) {
  const int64_t nc = (overlap ? 4 : 2) * (int64_t)c;
  int ks;
  int64_t sl;
  stream_split(nc, d, &ks, &sl);
  return (size_t)ks * (size_t)rows * (size_t)nc * sizeof(float);
}

// ------------------------------------------------------------------ attention

static int attn_path(const AttnArgs& a, bool dense) {
  if (a.q_dtype != ACT_BF16 || (a.kv_layout != ROW_BF16 && a.kv_layout != ROW_FP8)) return ATTN_GENERIC;
  if (!dense && a.k > ATTN_SIDX_CAP) return ATTN_GENERIC;
  // c = 512 with bf16 rows: two 32 KB stages and three key tiles exceed the
  // 160 KB of LDS, so that layout takes the generic kernel
  if (a.c == 512) {
    if (a.kv_layout != ROW_FP8) return ATTN_GENERIC;
    const bool ok = dense ? (a.nh == 16 || a.nh == 32 || a.nh == 64) : (a.nh == 32 || a.nh == 64);
    return ok ? ATTN_F8 : ATTN_GENERIC;
  }
  if (a.c == 128) {
    const bool ok = dense ? (a.nh == 16 || a.nh == 32 || a.nh == 64 || a.nh == 128)
                          : (a.nh == 32 || a.nh == 64 || a.nh == 128);
    return ok ? ATTN_MFMA : ATTN_GENERIC;
  }
  return ATTN_GENERIC;
}

// rows per block: one query (sparse) or 128 rows of queries sharing their keys
// (dense); c = 512 keeps 64 rows per block: Q^T and O^T of 32 rows x 256
// channels already take 192 registers per wave (all 512 channels of 32 rows
// in one wave would need 384 and spill)
static int rows_per_block(const AttnArgs& a, bool dense) {
  if (!dense) return a.nh;
  if (a.c >= 512) return a.nh < 64 ? 64 : a.nh;
  return a.nh > 128 ? a.nh : 128;
}

static int queries_per_group(const AttnArgs& a, bool dense) {
  if (attn_path(a, dense) == ATTN_GENERIC) return 1;
  const int q = rows_per_block(a, dense) / a.nh;
  return q < 1 ? 1 : q;
}

int64_t attn_group_slots(const AttnArgs& a, const int64_t* q_pos0, bool dense) {
  const int64_t qpw = queries_per_group(a, dense);
  int64_t best = 0;
  for (int64_t b = 0; b < a.B; ++b) {
    for (int64_t t0 = 0; t0 < a.nq; t0 += qpw) {
      const int64_t tl = (t0 + qpw < a.nq ? t0 + qpw : a.nq) - 1;
      const int64_t pf = q_pos0[b] + t0, pl = q_pos0[b] + tl;
      const int64_t ncomp = dense ? visible_count(pl, a.ratio, a.S) : a.k;
      int64_t wlen = 0;
      if (a.n_win > 0) {
        const int64_t wlo = pf - a.n_win + 1 > 0 ? pf - a.n_win + 1 : 0;
        wlen = pl - wlo + 1;
      }
      best = ncomp + wlen > best ? ncomp + wlen : best;
    }
  }
  return best;
}

AttnLaunchPlan attn_make_plan(const AttnArgs& a, bool dense, int64_t slots) {
  AttnLaunchPlan lp = {};
  lp.path = attn_path(a, dense);
  AttnPlan& pl = lp.pl;
  pl.dense = dense ? 1 : 0;
  pl.scale_log2 = a.scale * 1.4426950408889634f;
  if (lp.path == ATTN_GENERIC) {
    pl.qpw = 1;
    pl.units_per_b = a.nq;
    pl.chunk = 1 << 30;
    pl.max_splits = 1;
    lp.nrg = 0;
    lp.ws_bytes = 0;
    return lp;
  }
  const int rows = rows_per_block(a, dense);
  lp.nrg = rows / 32;
  pl.qpw = queries_per_group(a, dense);
  pl.units_per_b = (a.nq + pl.qpw - 1) / pl.qpw;
  // split the keys only when a sequence has few query groups.  The split size
  // depends on the key bound alone (never on the batch), so a sequence's
  // results do not depend on the batch.  The split count comes first and is
  // non-decreasing in the bound: up to 16 splits of at least 96 slots (a
  // decode query's 1152 sparse slots take 12 blocks of 3 key tiles), each split's bf16
  // partial (rows x c) small next to the rows it reads
  if (pl.units_per_b >= 32 || slots <= 0) {
    pl.chunk = 1 << 30;
    pl.max_splits = 1;
  } else {
    int64_t ms = (slots + 95) / 96;
    ms = ms < 1 ? 1 : (ms > ATTN_MAX_SPLITS ? ATTN_MAX_SPLITS : ms);
    const int64_t per = (slots + ms - 1) / ms;
    pl.chunk = (int)((per + 31) / 32 * 32);
    pl.max_splits = (int)ms;
  }
  if (pl.max_splits > 1) {
    const int64_t units = (a.B < MAXB ? a.B : MAXB) * pl.units_per_b;
    // per (unit, split, row): {m, l} in fp32 and the row's partial in bf16
    lp.ws_bytes = (size_t)units * pl.max_splits * pl.qpw * a.nh * (2 * sizeof(float) + (size_t)a.c * 2);
  }
  return lp;
}

size_t attn_workspace_bound(int64_t B, int64_t nq, int nh, int c, int64_t max_keys, bool dense) {
  if (B <= 0 || nq <= 0 || nh <= 0 || c <= 0) return 0;
  size_t best = 0;
  const int layouts[3] = {ROW_F32, ROW_BF16, ROW_FP8};
  for (int dt = ACT_F32; dt <= ACT_BF16; ++dt) {
    for (int li = 0; li < 3; ++li) {
      AttnArgs a = {};
      a.B = B; a.nq = nq; a.nh = nh; a.c = c; a.q_dtype = dt; a.kv_layout = layouts[li];
      a.k = dense ? 0 : (int)(max_keys < ATTN_SIDX_CAP ? max_keys : ATTN_SIDX_CAP);
      a.scale = 1.f;
      // a group's slots: one query's compressed entries and window rows, plus
      // the extra window positions its other queries reach back to
      const int64_t qpw = queries_per_group(a, dense);
      const int64_t span = qpw < nq ? qpw : nq;
      const int64_t slots = (max_keys > 0 ? max_keys : 0) + span - 1;
      const AttnLaunchPlan lp = attn_make_plan(a, dense, slots);
      best = lp.ws_bytes > best ? lp.ws_bytes : best;
    }
  }
  return best;
}

}  // namespace dsv4
