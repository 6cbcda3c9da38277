// Top-k selector (DeepSeek-V4 digest, 模块 B eq 17; jsqmd blog 第二阶段 Top-k稀疏选择).
//
// Every candidate becomes a unique 64-bit composite
//     (order-preserving uint32 key of the fp32 score) << 32  |  ~index
// so "score descending, ties to the lower index" is plain descending order of
// the composite, and the selected set is exactly { x >= T } for the k-th
// largest composite T.  T is found by an MSD radix select in LDS (12-bit
// digits, stopping as soon as a whole bin is taken), the winners are gathered
// and bitonic-sorted in LDS.
//
// Stage 1: one block per (row, part); a part is up to PART visible scores of
//          the row, staged once in LDS.  With one part the block writes the
//          final sorted indices; otherwise its k best composites go to the
//          workspace.
// Stage 2: one block per row merges the parts' candidates (at most 16384).
// Everything is exact integer work, so the result is bit-identical for any
// decomposition.
#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

constexpr int TK_THREADS = 1024;
constexpr int NBIN = 4096;
constexpr int MAX_CAND = 16384;

__device__ __forceinline__ uint32_t score_key(float x) {
  uint32_t u = __float_as_uint(x);
  if (u == 0x80000000u) u = 0u;                    // -0.0 ties with +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, uint32_t idx) {
  return ((uint64_t)key << 32) | (uint64_t)(~idx);
}

// inclusive block scan of one value per thread (1024 threads)
__device__ __forceinline__ uint32_t block_scan_incl(uint32_t v, uint32_t* wsum) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(v, o);
    if (lane >= o) v += n;
  }
  if (lane == 63) wsum[w] = v;
  __syncthreads();
  if (w == 0) {
    uint32_t x = lane < (TK_THREADS / 64) ? wsum[lane] : 0u;
    for (int o = 1; o < 16; o <<= 1) {
      const uint32_t n = __shfl_up(x, o);
      if (lane >= o) x += n;
    }
    if (lane < 16) wsum[lane] = x;
  }
  __syncthreads();
  const uint32_t r = v + (w ? wsum[w - 1] : 0u);
  __syncthreads();
  return r;
}

struct SelState {
  uint64_t prefix;
  uint32_t remaining;
  uint32_t done;
  uint32_t bin;
  uint32_t above;
  uint32_t cnt;
};

// Find T with #{x >= T} == need among the composites produced by get(i),
// i < N (need >= 1, need <= N, composites unique and non-zero).
template <typename Get>
__device__ uint64_t radix_threshold(Get get, int N, uint32_t need, uint32_t* hist, uint32_t* wsum,
                                    SelState* st) {
  if (threadIdx.x == 0) { st->prefix = 0; st->remaining = need; st->done = 0; }
  __syncthreads();
  int shift = 64;
  for (int level = 0; level < 6; ++level) {
    const int width = level < 5 ? 12 : 4;
    shift -= width;
    for (int i = threadIdx.x; i < NBIN; i += TK_THREADS) hist[i] = 0;
    __syncthreads();
    const uint64_t prefix = st->prefix;
    const int hs = shift + width;
    for (int i = threadIdx.x; i < N; i += TK_THREADS) {
      const uint64_t x = get(i);
      if (hs >= 64 || (x >> hs) == (prefix >> hs))
        atomicAdd(&hist[(uint32_t)(x >> shift) & (NBIN - 1)], 1u);
    }
    __syncthreads();
    // thread t owns bins [NBIN - 4(t+1), NBIN - 4t), scanned from the top
    uint32_t c4[4];
    uint32_t loc = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) { c4[q] = hist[NBIN - 1 - (4 * threadIdx.x + q)]; loc += c4[q]; }
    const uint32_t incl = block_scan_incl(loc, wsum);
    const uint32_t rem = st->remaining;
    uint32_t above = incl - loc;
    if (above < rem && rem <= incl) {
      for (int q = 0; q < 4; ++q) {
        if (above + c4[q] >= rem) {
          st->bin = NBIN - 1 - (4 * threadIdx.x + q);
          st->above = above;
          st->cnt = c4[q];
          break;
        }
        above += c4[q];
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      st->prefix |= (uint64_t)st->bin << shift;
      st->remaining -= st->above;
      if (st->cnt == st->remaining) st->done = 1;
    }
    __syncthreads();
    if (st->done) break;
  }
  return st->prefix;
}

// descending bitonic sort of n (power of two) composites in LDS
__device__ void bitonic_desc(uint64_t* buf, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += TK_THREADS) {
        const int pos = 2 * i - (i & (stride - 1));
        const int par = pos + stride;
        const bool desc = (pos & size) == 0;
        const uint64_t x = buf[pos], y = buf[par];
        if ((x < y) == desc) { buf[pos] = y; buf[par] = x; }
      }
      __syncthreads();
    }
  }
}

struct TopkArgs {
  const float* scores;
  int64_t nq, S;
  int m, k;
  int part;          // scores per stage-1 part
  int nparts;
  int32_t* idx;      // [rows, k]
  uint64_t* cand;    // [rows, nparts, k] (nparts > 1)
};

__device__ __forceinline__ int pow2_ceil(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

// dynamic LDS: part * 4 (keys) | NBIN * 4 | pow2(k) * 8
__global__ __launch_bounds__(TK_THREADS) void topk_stage1(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t wsum[16];
  __shared__ SelState st;
  __shared__ uint32_t cnt;
  uint32_t* keys = reinterpret_cast<uint32_t*>(smem);
  uint32_t* hist = keys + a.part;
  uint64_t* out = reinterpret_cast<uint64_t*>(hist + NBIN);

  const int64_t row = (int64_t)blockIdx.x;         // row within this launch's batch slice
  const int pidx = blockIdx.y;
  const int64_t bl = row / a.nq, t = row % a.nq;
  const int64_t grow = (b0 + bl) * a.nq + t;       // global row
  const int64_t nv = visible_count(pt.q_pos0[bl] + t, a.m, a.S);
  const int64_t lo = (int64_t)pidx * a.part;
  const int N = (int)(nv - lo < 0 ? 0 : (nv - lo < a.part ? nv - lo : a.part));
  const uint32_t need = (uint32_t)(N < a.k ? N : a.k);
  const float* src = a.scores + grow * a.S + lo;

  for (int i = threadIdx.x; i < N; i += TK_THREADS) keys[i] = score_key(src[i]);
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();

  uint64_t T = 1;
  auto get = [&](int i) { return composite(keys[i], (uint32_t)(lo + i)); };
  if (need > 0 && need < (uint32_t)N) T = radix_threshold(get, N, need, hist, wsum, &st);
  for (int i = threadIdx.x; i < N; i += TK_THREADS) {
    const uint64_t x = get(i);
    if (need > 0 && x >= T) {
      const uint32_t at = atomicAdd(&cnt, 1u);
      if (at < need) out[at] = x;
    }
  }
  __syncthreads();
  if (a.nparts == 1) {
    const int n2 = pow2_ceil(a.k);
    for (int i = need + threadIdx.x; i < n2; i += TK_THREADS) out[i] = 0;
    __syncthreads();
    bitonic_desc(out, n2);
    for (int i = threadIdx.x; i < a.k; i += TK_THREADS)
      a.idx[grow * a.k + i] = i < (int)need ? (int32_t)(~(uint32_t)out[i]) : -1;
  } else {
    uint64_t* dst = a.cand + (row * a.nparts + pidx) * a.k;   // launch-local row
    for (int i = threadIdx.x; i < a.k; i += TK_THREADS) dst[i] = i < (int)need ? out[i] : 0;
  }
}

// dynamic LDS: nparts*k * 8 | NBIN * 4 | pow2(k) * 8
__global__ __launch_bounds__(TK_THREADS) void topk_stage2(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ uint32_t wsum[16];
  __shared__ SelState st;
  __shared__ uint32_t cnt;
  const int NC = a.nparts * a.k;
  uint64_t* cand = reinterpret_cast<uint64_t*>(smem);
  uint32_t* hist = reinterpret_cast<uint32_t*>(cand + NC);
  uint64_t* out = reinterpret_cast<uint64_t*>(hist + NBIN);

  const int64_t row = (int64_t)blockIdx.x;
  const int64_t bl = row / a.nq, t = row % a.nq;
  const int64_t grow = (b0 + bl) * a.nq + t;
  const int64_t nv = visible_count(pt.q_pos0[bl] + t, a.m, a.S);
  uint32_t valid = 0;
  for (int p = 0; p < a.nparts; ++p) {
    const int64_t len = nv - (int64_t)p * a.part;
    valid += (uint32_t)(len <= 0 ? 0 : (len < a.k ? len : a.k));
  }
  const uint32_t need = valid < (uint32_t)a.k ? valid : (uint32_t)a.k;
  const uint64_t* src = a.cand + row * NC;
  for (int i = threadIdx.x; i < NC; i += TK_THREADS) cand[i] = src[i];
  if (threadIdx.x == 0) cnt = 0;
  __syncthreads();
  uint64_t T = 1;
  auto get = [&](int i) { return cand[i]; };
  if (need > 0 && need < valid) T = radix_threshold(get, NC, need, hist, wsum, &st);
  for (int i = threadIdx.x; i < NC; i += TK_THREADS) {
    const uint64_t x = cand[i];
    if (need > 0 && x != 0 && x >= T) {
      const uint32_t at = atomicAdd(&cnt, 1u);
      if (at < need) out[at] = x;
    }
  }
  __syncthreads();
  const int n2 = pow2_ceil(a.k);
  for (int i = need + threadIdx.x; i < n2; i += TK_THREADS) out[i] = 0;
  __syncthreads();
  bitonic_desc(out, n2);
  for (int i = threadIdx.x; i < a.k; i += TK_THREADS)
    a.idx[grow * a.k + i] = i < (int)need ? (int32_t)(~(uint32_t)out[i]) : -1;
}

static void topk_plan(int64_t rows, int64_t S, int k, int* part, int* nparts) {
  int p = k <= 1024 ? 32768 : 16384;
  if (rows < 256 && S > 16384 && k <= 1024) p = 16384;   // more blocks for few rows
  int fit = 4096;                                         // short rows: a smaller LDS stage
  while (fit < S && fit < p) fit <<= 1;
  p = fit < p ? fit : p;
  *part = p;
  *nparts = (int)((S + p - 1) / p);
}

size_t topk_workspace_bytes(int64_t rows, int64_t S, int k) {
  int part, nparts;
  topk_plan(rows, S, k, &part, &nparts);
  return nparts > 1 ? (size_t)rows * nparts * k * sizeof(uint64_t) : 0;
}

bool topk_supported(int64_t rows, int64_t S, int k) {
  int part, nparts;
  topk_plan(rows, S, k, &part, &nparts);
  return k >= 1 && k <= 4096 && (nparts == 1 || (int64_t)nparts * k <= MAX_CAND);
}

hipError_t launch_topk(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                       const int64_t* q_pos0, int k, int32_t* idx, void* ws, hipStream_t s) {
  if (B <= 0 || nq <= 0) return hipSuccess;
  TopkArgs a;
  a.scores = scores; a.nq = nq; a.S = S; a.m = m; a.k = k; a.idx = idx;
  topk_plan((B < MAXB ? B : MAXB) * nq, S, k, &a.part, &a.nparts);
  a.cand = reinterpret_cast<uint64_t*>(ws);
  const int n2 = [&] { int p = 1; while (p < k) p <<= 1; return p; }();
  const size_t lds1 = (size_t)a.part * 4 + NBIN * 4 + (size_t)n2 * 8;
  const size_t lds2 = (size_t)a.nparts * k * 8 + NBIN * 4 + (size_t)n2 * 8;
  hipError_t e = hipFuncSetAttribute((const void*)topk_stage1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  if (e != hipSuccess) return e;
  if (a.nparts > 1) {
    e = hipFuncSetAttribute((const void*)topk_stage2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
    if (e != hipSuccess) return e;
  }
  for (int64_t b0 = 0; b0 < B; b0 += MAXB) {
    const int nb = (int)(B - b0 < MAXB ? B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
    hipLaunchKernelGGL(topk_stage1, dim3((unsigned)(nb * nq), (unsigned)a.nparts), dim3(TK_THREADS), lds1, s,
                       a, pt, (int)b0);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.nparts > 1) {
      hipLaunchKernelGGL(topk_stage2, dim3((unsigned)(nb * nq)), dim3(TK_THREADS), lds2, s, a, pt, (int)b0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

}  // namespace dsv4
