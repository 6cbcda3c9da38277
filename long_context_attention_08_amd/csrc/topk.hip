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
// k <= 1024, streaming: one block per (row, part) reads its scores once from
//          HBM.  A running threshold tau (a composite no larger than the k-th
//          largest seen so far) rejects almost every score with one float
//          compare; the survivors go to an LDS candidate buffer, which is cut
//          back to its k largest (exact radix select, first digit at the
//          highest bit where the candidates differ) whenever a step could
//          overflow it.  A rejected score is below k kept ones, so it cannot
//          be selected.
// k > 1024: stage 1, one block per (row, part); a part is up to PART visible
//          scores staged once in LDS and radix-selected there.
// Either way, with one part the block writes the final sorted indices;
// otherwise its k best composites go to the workspace and stage 2 (one block
// per row) merges the parts' candidates (at most 16384).  Everything is exact
// integer work, so the result is bit-identical for any decomposition.
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

// descending bitonic sort of n (power of two) composites in LDS, NT threads
template <int NT = TK_THREADS>
__device__ void bitonic_desc(uint64_t* buf, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += NT) {
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

struct HsMeta {
  int bstar;         // threshold bin (-1: every visible score is taken)
  uint32_t above;    // visible keys in bins above bstar (all winners)
  uint32_t inbin;    // visible keys in bin bstar
  uint32_t need;     // min(k, visible)
};

struct TopkArgs {
  const float* scores;
  int64_t nq, S;
  int m, k;
  int part;          // scores per stage-1 part
  int nparts;
  int32_t* idx;      // [rows, k]
  uint64_t* cand;    // [rows, nparts, k] (nparts > 1)
  // histogram select (few long rows)
  uint32_t* hsuf;    // [rows, nparts, HS_BIN] suffix counts per part
  uint32_t* hoff;    // [rows, nparts, 2] write offsets (winners, bin candidates)
  HsMeta* hmeta;     // [rows]
  uint64_t* hwin;    // [rows, k] winners above the threshold bin
  uint64_t* hcand;   // [rows, HS_CAP] keys of the threshold bin
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

// ------------------------------------------------------------------ streaming select (k <= 1024)

constexpr int SK_NT = 256;                  // threads per block
constexpr int SK_U = 2;                     // float4 loads per thread and step
constexpr int SK_STEP = SK_NT * 4 * SK_U;   // scores per step
// candidate slots of the streaming kernel (>= SK_STEP + k): 28 KB, so that
// four blocks share a CU; a block's loop is latency-bound (a barrier and a
// ballot append per step), and more blocks per CU raise the HBM rate
constexpr int SK_CAP = 3584;
constexpr int HS_CAP = 8192;                // threshold-bin candidates of the histogram select
constexpr int SK_BIN = 2048;                // 11-bit digits
constexpr int SK_KMAX = 1024;

template <int CAP>
struct SkSharedT {
  uint64_t cand[CAP];
  union {                                   // the histogram is dead once the gather starts
    uint64_t out[SK_KMAX];
    uint32_t hist[SK_BIN];
  };
  uint64_t rmin[SK_NT / 64], rmax[SK_NT / 64];
  uint32_t wsum[SK_NT / 64];
  uint32_t cnt, cnt2;
  uint32_t sel_bin, sel_above, sel_cnt;
};
using SkShared = SkSharedT<SK_CAP>;     // streaming select
using HsShared = SkSharedT<HS_CAP>;     // last step of the histogram select
static_assert(SK_CAP >= SK_STEP + SK_KMAX, "a step must fit next to the k kept candidates");

// Barrier for LDS traffic only (waits for this wave's LDS operations): unlike
// __syncthreads() it carries no memory fence, so score loads in flight stay
// in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);     // lgkmcnt(0)
  __builtin_amdgcn_s_barrier();
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int o) {
  const uint32_t lo = __shfl_xor((uint32_t)v, o), hi = __shfl_xor((uint32_t)(v >> 32), o);
  return ((uint64_t)hi << 32) | lo;
}

// Descending bitonic sort of the 1024 composites in buf (LDS), SK_NT = 256
// threads, element e = 4 t + j held in register j of thread t: strides 1 and
// 2 compare within a thread, strides 4 .. 128 with the lane t ^ (stride / 4)
// of the same wave, and only strides 256 and 512 go through LDS.  The result
// is written back to buf in order.
__device__ void bitonic1024_desc(uint64_t* buf) {
  static_assert(SK_NT == 256, "4 elements per thread");
  const int t = threadIdx.x;
  uint64_t v[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) v[j] = buf[4 * t + j];
  __syncthreads();
  for (int size = 2; size <= 1024; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride < 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int pj = j ^ stride;
          if (pj > j) {
            const int e = 4 * t + j;
            const bool desc = (e & size) == 0;
            const uint64_t x = v[j], y = v[pj];
            if ((x < y) == desc) { v[j] = y; v[pj] = x; }
          }
        }
      } else if (stride < 256) {
        const int lo = stride >> 2;                  // partner lane distance
        const bool lower = (t & lo) == 0;            // this thread holds the lower index of each pair
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * t + j;
          const bool desc = (e & size) == 0;
          const uint64_t y = shfl_xor_u64(v[j], lo);
          const uint64_t mx = v[j] > y ? v[j] : y, mn = v[j] > y ? y : v[j];
          v[j] = (lower == desc) ? mx : mn;
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) buf[4 * t + j] = v[j];
        __syncthreads();
        const int pt = t ^ (stride >> 2);
        const bool lower = (t & (stride >> 2)) == 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int e = 4 * t + j;
          const bool desc = (e & size) == 0;
          const uint64_t y = buf[4 * pt + j];
          const uint64_t mx = v[j] > y ? v[j] : y, mn = v[j] > y ? y : v[j];
          v[j] = (lower == desc) ? mx : mn;
        }
        __syncthreads();
      }
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) buf[4 * t + j] = v[j];
  __syncthreads();
}

// exclusive prefix over the SK_NT threads of a per-thread count; *total gets the sum
__device__ __forceinline__ uint32_t sk_scan_excl(uint32_t v, uint32_t* wsum, uint32_t* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t x = v;
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t n = __shfl_up(x, o);
    if (lane >= o) x += n;
  }
  if (lane == 63) wsum[w] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < SK_NT / 64; ++i) {
    const uint32_t ws = wsum[i];
    before += i < w ? ws : 0u;
    all += ws;
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

// the composite T with #{cand[i] >= T, i < n} == need (1 <= need <= n, unique, non-zero)
template <class Sh>
__device__ uint64_t sk_select(Sh& sh, int n, uint32_t need) {
  uint64_t mn = ~0ull, mx = 0;
  for (int i = threadIdx.x; i < n; i += SK_NT) {
    const uint64_t x = sh.cand[i];
    mn = x < mn ? x : mn;
    mx = x > mx ? x : mx;
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t a = shfl_xor_u64(mn, o), b = shfl_xor_u64(mx, o);
    mn = a < mn ? a : mn;
    mx = b > mx ? b : mx;
  }
  if ((threadIdx.x & 63) == 0) { sh.rmin[threadIdx.x >> 6] = mn; sh.rmax[threadIdx.x >> 6] = mx; }
  __syncthreads();
  mn = sh.rmin[0];
  mx = sh.rmax[0];
#pragma unroll
  for (int i = 1; i < SK_NT / 64; ++i) {
    mn = sh.rmin[i] < mn ? sh.rmin[i] : mn;
    mx = sh.rmax[i] > mx ? sh.rmax[i] : mx;
  }
  if (need >= (uint32_t)n) return mn;          // everything is taken
  // bits above the highest differing one are common to all candidates
  const int hb = 63 - __clzll(mn ^ mx);
  int shift = hb + 1;
  uint64_t prefix = shift >= 64 ? 0ull : (mn >> shift) << shift;
  uint32_t remaining = need;
  for (;;) {
    const int width = shift < 11 ? shift : 11;
    shift -= width;
    const int top = shift + width;               // bits at and above `top` must match prefix
    for (int i = threadIdx.x; i < SK_BIN; i += SK_NT) sh.hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += SK_NT) {
      const uint64_t x = sh.cand[i];
      if (top >= 64 || (x >> top) == (prefix >> top))
        atomicAdd(&sh.hist[(uint32_t)(x >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    // thread t owns the 8 bins [SK_BIN - 8(t+1), SK_BIN - 8t), scanned from the top
    constexpr int PER = SK_BIN / SK_NT;
    uint32_t c[PER];
    uint32_t loc = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) { c[q] = sh.hist[SK_BIN - 1 - (PER * threadIdx.x + q)]; loc += c[q]; }
    uint32_t total;
    uint32_t above = sk_scan_excl(loc, sh.wsum, &total);
    if (above < remaining && remaining <= above + loc) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (above < remaining && remaining <= above + c[q]) {
          sh.sel_bin = SK_BIN - 1 - (PER * threadIdx.x + q);
          sh.sel_above = above;
          sh.sel_cnt = c[q];
        }
        above += c[q];
      }
    }
    __syncthreads();
    const uint32_t bin = sh.sel_bin, ab = sh.sel_above, cb = sh.sel_cnt;
    __syncthreads();
    prefix |= (uint64_t)bin << shift;
    remaining -= ab;
    if (cb == remaining || shift == 0) return prefix;   // the whole bin is taken
  }
}

// keep the `need` candidates >= T in sh.out (any order); returns through sh.out
template <class Sh>
__device__ void sk_gather(Sh& sh, int n, uint64_t T) {
  if (threadIdx.x == 0) sh.cnt2 = 0;
  __syncthreads();
  for (int i = threadIdx.x; i < n; i += SK_NT) {
    const uint64_t x = sh.cand[i];
    if (x >= T) {
      const uint32_t at = atomicAdd(&sh.cnt2, 1u);
      if (at < SK_KMAX) sh.out[at] = x;
    }
  }
  __syncthreads();
}

// dynamic LDS: sizeof(SkShared).  VEC: every part starts 16-byte aligned, so
// whole steps are read with float4 loads (the last, partial step with
// clamped scalar loads).
template <bool VEC>
__global__ __launch_bounds__(SK_NT) void topk_stream(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  SkShared& sh = *reinterpret_cast<SkShared*>(smem);
  const int64_t row = (int64_t)blockIdx.x;         // row within this launch's batch slice
  const int pidx = blockIdx.y;
  const int64_t bl = row / a.nq, t = row % a.nq;
  const int64_t grow = (b0 + bl) * a.nq + t;       // global row
  const int64_t nv = visible_count(pt.q_pos0[bl] + t, a.m, a.S);
  const int64_t lo = (int64_t)pidx * a.part;
  const int N = (int)(nv - lo < 0 ? 0 : (nv - lo < a.part ? nv - lo : a.part));
  const uint32_t need = (uint32_t)(N < a.k ? N : a.k);
  const float* src = a.scores + grow * a.S + lo;
  if (threadIdx.x == 0) sh.cnt = 0;

  uint64_t tau = 0;                  // composites must exceed tau to enter
  float tauf = __uint_as_float(0xFFFFFFFFu);   // score of tau's key (NaN while tau = 0)
  typedef float f4 __attribute__((ext_vector_type(4)));
  // loads without per-lane branches, so that the compiler's waits stay per buffer
  auto load_vec = [&](int i0, f4 (&d)[SK_U]) {     // a whole step, i0 + SK_STEP <= N
#pragma unroll
    for (int u = 0; u < SK_U; ++u)
      d[u] = *reinterpret_cast<const f4*>(src + i0 + (u * SK_NT + (int)threadIdx.x) * 4);
  };
  auto load_sca = [&](int i0, f4 (&d)[SK_U]) {     // indices past N read element N-1 (masked later)
#pragma unroll
    for (int u = 0; u < SK_U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = i0 + (u * SK_NT + (int)threadIdx.x) * 4 + j;
        d[u][j] = src[e < N ? e : N - 1];
      }
  };
  auto load = [&](int i0, f4 (&d)[SK_U]) {
    if (VEC) load_vec(i0, d);
    else load_sca(i0, d);
  };
  // cut the buffer back to its `need` largest and raise tau
  auto compact = [&]() {
    const int n = (int)sh.cnt;
    const uint64_t T = sk_select(sh, n, need);
    sk_gather(sh, n, T);
    for (int i = threadIdx.x; i < (int)need; i += SK_NT) sh.cand[i] = sh.out[i];
    if (threadIdx.x == 0) sh.cnt = need;
    __syncthreads();
    tau = T;
    const uint32_t th = (uint32_t)(T >> 32);
    tauf = __uint_as_float((th & 0x80000000u) ? (th ^ 0x80000000u) : ~th);
  };
  auto process = [&](int i0, const f4 (&d)[SK_U]) {
    lds_barrier();                                     // every append of the last step is in
    if (sh.cnt > (uint32_t)(SK_CAP - SK_STEP)) compact();
    // survivors: scores not below tauf, then the exact composite test
    uint64_t keep[SK_U * 4];
    bool anyk = false;
#pragma unroll
    for (int u = 0; u < SK_U; ++u)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = i0 + (u * SK_NT + (int)threadIdx.x) * 4 + j;
        const float x = d[u][j];
        keep[u * 4 + j] = 0;
        if (e < N && !(x < tauf)) {
          const uint64_t c = composite(score_key(x), (uint32_t)(lo + e));
          if (c > tau) keep[u * 4 + j] = c;
        }
        anyk |= keep[u * 4 + j] != 0;
      }
    // wave-local append: one LDS atomic per wave, positions from ballots
    if (__ballot(anyk) != 0) {
      uint64_t bal[SK_U * 4];
      uint32_t total = 0;
#pragma unroll
      for (int i = 0; i < SK_U * 4; ++i) {
        bal[i] = __ballot(keep[i] != 0);
        total += (uint32_t)__popcll(bal[i]);
      }
      uint32_t base = 0;
      if ((threadIdx.x & 63) == 0) base = atomicAdd(&sh.cnt, total);
      base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
      for (int i = 0; i < SK_U * 4; ++i) {
        if (keep[i] != 0)
          sh.cand[base + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal[i] >> 32),
                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)bal[i], 0u))] = keep[i];
        base += (uint32_t)__popcll(bal[i]);
      }
    }
  };

  // four register buffers in rotation: three steps of loads in flight; a
  // partial last step follows with scalar loads.
  // Every load is issued unconditionally (steps past the end re-read the last
  // whole step, never processed twice), so the compiler's per-buffer wait
  // counts stay exact.  The rotation covers whole steps only.
  constexpr int ST = SK_STEP;
  const int NM = N / ST * ST;
  if (NM > 0) {
    const int last = NM - ST;
    auto cl = [&](int i) { return i < last ? i : last; };
    f4 A[SK_U], B[SK_U], C[SK_U], D[SK_U];
    load(0, A);
    load(cl(ST), B);
    load(cl(2 * ST), C);
    for (int i0 = 0; i0 < NM; i0 += 4 * ST) {
      load(cl(i0 + 3 * ST), D);
      process(i0, A);
      load(cl(i0 + 4 * ST), A);
      if (i0 + ST < NM) process(i0 + ST, B);
      load(cl(i0 + 5 * ST), B);
      if (i0 + 2 * ST < NM) process(i0 + 2 * ST, C);
      load(cl(i0 + 6 * ST), C);
      if (i0 + 3 * ST < NM) process(i0 + 3 * ST, D);
    }
  }
  if (NM < N) {
    f4 T[SK_U];
    load_sca(NM, T);
    process(NM, T);
  }
  __syncthreads();
  // final selection of the `need` largest, sorted descending
  const int n = (int)sh.cnt;
  if (need > 0) {
    const uint64_t T = sk_select(sh, n, need);
    sk_gather(sh, n, T);
  }
  if (a.nparts == 1) {
    const int n2 = pow2_ceil(a.k) > 256 ? SK_KMAX : pow2_ceil(a.k);
    for (int i = need + threadIdx.x; i < n2; i += SK_NT) sh.out[i] = 0;
    __syncthreads();
    if (n2 == SK_KMAX) bitonic1024_desc(sh.out);
    else bitonic_desc<SK_NT>(sh.out, n2);
    for (int i = threadIdx.x; i < a.k; i += SK_NT)
      a.idx[grow * a.k + i] = i < (int)need ? (int32_t)(~(uint32_t)sh.out[i]) : -1;
  } else {
    uint64_t* dst = a.cand + (row * a.nparts + pidx) * a.k;   // launch-local row
    for (int i = threadIdx.x; i < a.k; i += SK_NT) dst[i] = i < (int)need ? sh.out[i] : 0;
  }
}

// ------------------------------------------------------------------ histogram select (few long rows, k <= 1024)
// Decode has a handful of rows of 2^18 scores.  Each row is cut into parts and
// processed in four launches, each a plain pass:
//   1. per part: a 2048-bin histogram of the top 11 key bits, stored as suffix
//      counts (keys at or above each bin);
//   2. per row: the threshold bin b* (the highest bin whose suffix count
//      reaches min(k, visible)), how many keys lie above it and in it, and
//      every part's write offsets into the winner and candidate lists;
//   3. per part: keys above b* go to the winner list, keys in b* to the
//      candidate list, as composites;
//   4. per row: the candidates are cut to the missing count by the exact
//      radix select, and the k winners are bitonic-sorted.  When b* holds more
//      keys than the candidate list (heavy ties), the select runs over the row
//      in global memory instead.
// The selected set is the same exact set as on every other path.
constexpr int HS_BIN = 2048;
constexpr int HS_PER = HS_BIN / SK_NT;     // bins per thread

__device__ __forceinline__ int64_t hs_row(const TopkArgs& a, const PosTable& pt, int b0, int64_t row,
                                          int64_t* nv) {
  const int64_t bl = row / a.nq, t = row % a.nq;
  *nv = visible_count(pt.q_pos0[bl] + t, a.m, a.S);
  return (b0 + bl) * a.nq + t;
}

__global__ __launch_bounds__(SK_NT) void topk_h_hist(TopkArgs a, PosTable pt, int b0) {
  __shared__ uint32_t h[HS_BIN];
  __shared__ uint32_t wsum[SK_NT / 64];
  const int64_t row = blockIdx.y;
  const int p = blockIdx.x;
  int64_t nv;
  const int64_t grow = hs_row(a, pt, b0, row, &nv);
  const int64_t s0 = (int64_t)p * a.part, s1 = s0 + a.part < nv ? s0 + a.part : nv;
  for (int i = threadIdx.x; i < HS_BIN; i += SK_NT) h[i] = 0;
  __syncthreads();
  const float* src = a.scores + grow * a.S;
  // eight loads in flight per thread (clamped indices, used only when in range)
  for (int64_t base = s0; base < s1; base += 8 * SK_NT) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = base + u * SK_NT + threadIdx.x;
      x[u] = src[s < s1 ? s : s1 - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (base + u * SK_NT + threadIdx.x < s1) atomicAdd(&h[score_key(x[u]) >> 21], 1u);
  }
  __syncthreads();
  uint32_t c[HS_PER];
  uint32_t loc = 0;
#pragma unroll
  for (int q = 0; q < HS_PER; ++q) { c[q] = h[HS_PER * threadIdx.x + q]; loc += c[q]; }
  uint32_t total;
  const uint32_t before = sk_scan_excl(loc, wsum, &total);
  uint32_t acc = total - before - loc;       // keys in the bins above this thread's range
  uint32_t* dst = a.hsuf + (row * a.nparts + p) * HS_BIN + HS_PER * threadIdx.x;
#pragma unroll
  for (int q = HS_PER - 1; q >= 0; --q) {
    acc += c[q];
    dst[q] = acc;
  }
}

__global__ __launch_bounds__(SK_NT) void topk_h_thresh(TopkArgs a, PosTable pt, int b0) {
  __shared__ uint32_t wsum[SK_NT / 64];
  __shared__ int s_b;
  __shared__ uint32_t s_t0[SK_NT + 1];
  static_assert(HS_PER == 8, "two 16-byte loads per part and thread");
  const int64_t row = blockIdx.x;
  int64_t nv;
  hs_row(a, pt, b0, row, &nv);
  const uint32_t need = (uint32_t)(nv < a.k ? nv : a.k);
  const uint32_t* suf = a.hsuf + row * a.nparts * HS_BIN;
  const bool cut = need < (uint64_t)nv;
  // total suffix counts of this thread's 8 bins over all parts (loads in flight together)
  uint32_t tot[HS_PER];
#pragma unroll
  for (int q = 0; q < HS_PER; ++q) tot[q] = 0;
  if (cut) {
    const u32x4* sp = reinterpret_cast<const u32x4*>(suf) + 2 * threadIdx.x;
#pragma unroll 8
    for (int pp = 0; pp < a.nparts; ++pp) {
      const u32x4 x0 = sp[pp * (HS_BIN / 4)], x1 = sp[pp * (HS_BIN / 4) + 1];
#pragma unroll
      for (int q = 0; q < 4; ++q) { tot[q] += x0[q]; tot[4 + q] += x1[q]; }
    }
  }
  s_t0[threadIdx.x] = tot[0];
  if (threadIdx.x == 0) { s_t0[SK_NT] = 0; s_b = -1; }
  __syncthreads();
  if (cut) {
    // exactly one bin has suffix >= need while the next one up has less
    const uint32_t nxt = s_t0[threadIdx.x + 1];
#pragma unroll
    for (int q = 0; q < HS_PER; ++q) {
      const uint32_t up = q + 1 < HS_PER ? tot[q + 1] : nxt;
      if (tot[q] >= need && up < need) s_b = HS_PER * threadIdx.x + q;
    }
  }
  __syncthreads();
  const int bstar = s_b;
  uint32_t ca = 0, cb = 0;
  if ((int)threadIdx.x < a.nparts) {
    const uint32_t* sp = suf + threadIdx.x * HS_BIN;
    ca = bstar + 1 < HS_BIN ? sp[bstar + 1] : 0u;
    cb = bstar >= 0 ? sp[bstar] - ca : 0u;
  }
  uint32_t ta, tb;
  const uint32_t ea = sk_scan_excl(ca, wsum, &ta);
  const uint32_t eb = sk_scan_excl(cb, wsum, &tb);
  if ((int)threadIdx.x < a.nparts) {
    a.hoff[(row * a.nparts + threadIdx.x) * 2] = ea;
    a.hoff[(row * a.nparts + threadIdx.x) * 2 + 1] = eb;
  }
  if (threadIdx.x == 0) a.hmeta[row] = HsMeta{bstar, ta, tb, need};
}

__global__ __launch_bounds__(SK_NT) void topk_h_compact(TopkArgs a, PosTable pt, int b0) {
  __shared__ uint32_t na, nb;
  const int64_t row = blockIdx.y;
  const int p = blockIdx.x;
  int64_t nv;
  const int64_t grow = hs_row(a, pt, b0, row, &nv);
  const HsMeta mt = a.hmeta[row];
  if (mt.need == 0) return;
  const uint32_t offa = a.hoff[(row * a.nparts + p) * 2], offb = a.hoff[(row * a.nparts + p) * 2 + 1];
  if (threadIdx.x == 0) { na = 0; nb = 0; }
  __syncthreads();
  const int64_t s0 = (int64_t)p * a.part, s1 = s0 + a.part < nv ? s0 + a.part : nv;
  const float* src = a.scores + grow * a.S;
  uint64_t* win = a.hwin + row * a.k;
  uint64_t* cand = a.hcand + row * HS_CAP;
  for (int64_t base = s0; base < s1; base += 8 * SK_NT) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = base + u * SK_NT + threadIdx.x;
      x[u] = src[s < s1 ? s : s1 - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t s = base + u * SK_NT + threadIdx.x;
      if (s >= s1) continue;
      const uint32_t key = score_key(x[u]);
      const int bin = (int)(key >> 21);
      if (bin > mt.bstar) {
        win[offa + atomicAdd(&na, 1u)] = composite(key, (uint32_t)s);
      } else if (bin == mt.bstar) {
        const uint32_t at = offb + atomicAdd(&nb, 1u);
        if (at < (uint32_t)HS_CAP) cand[at] = composite(key, (uint32_t)s);
      }
    }
  }
}

// global -> LDS copy of n composites, eight loads in flight per thread
__device__ __forceinline__ void hs_copy(uint64_t* dst, const uint64_t* src, uint32_t n) {
  for (uint32_t base = 0; base < n; base += 8 * SK_NT) {
    uint64_t x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = base + u * SK_NT + threadIdx.x;
      x[u] = src[i < n ? i : n - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t i = base + u * SK_NT + threadIdx.x;
      if (i < n) dst[i] = x[u];
    }
  }
}

// dynamic LDS: sizeof(HsShared)
__global__ __launch_bounds__(SK_NT) void topk_h_finish(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  HsShared& sh = *reinterpret_cast<HsShared*>(smem);
  const int64_t row = blockIdx.x;
  int64_t nv;
  const int64_t grow = hs_row(a, pt, b0, row, &nv);
  const HsMeta mt = a.hmeta[row];
  const uint32_t need = mt.need, nab = mt.above;
  const uint32_t needb = need - nab;                 // to take from bin b*
  const bool spill = mt.inbin > (uint32_t)HS_CAP;
  const float* src = a.scores + grow * a.S;
  const uint64_t pre = (uint64_t)(uint32_t)mt.bstar << 53;   // composites of bin b* start with it
  uint64_t T = ~0ull;
  if (needb > 0 && !spill) {
    hs_copy(sh.cand, a.hcand + row * HS_CAP, mt.inbin);
    __syncthreads();
    T = sk_select(sh, (int)mt.inbin, needb);
  } else if (needb > 0) {
    // exact MSD radix select over the row's keys of bin b*, read from global memory
    uint64_t prefix = pre;
    uint32_t remaining = needb;
    int shift = 53;
    for (;;) {
      const int width = shift < 11 ? shift : 11;
      shift -= width;
      const int top = shift + width;
      for (int i = threadIdx.x; i < SK_BIN; i += SK_NT) sh.hist[i] = 0;
      __syncthreads();
      for (int64_t s = threadIdx.x; s < nv; s += SK_NT) {
        const uint64_t x = composite(score_key(src[s]), (uint32_t)s);
        if ((x >> top) == (prefix >> top)) atomicAdd(&sh.hist[(uint32_t)(x >> shift) & ((1u << width) - 1u)], 1u);
      }
      __syncthreads();
      uint32_t c[HS_PER];
      uint32_t loc = 0;
#pragma unroll
      for (int q = 0; q < HS_PER; ++q) { c[q] = sh.hist[SK_BIN - 1 - (HS_PER * threadIdx.x + q)]; loc += c[q]; }
      uint32_t total;
      uint32_t above = sk_scan_excl(loc, sh.wsum, &total);
      if (above < remaining && remaining <= above + loc) {
#pragma unroll
        for (int q = 0; q < HS_PER; ++q) {
          if (above < remaining && remaining <= above + c[q]) {
            sh.sel_bin = SK_BIN - 1 - (HS_PER * threadIdx.x + q);
            sh.sel_above = above;
            sh.sel_cnt = c[q];
          }
          above += c[q];
        }
      }
      __syncthreads();
      const uint32_t bin = sh.sel_bin, ab = sh.sel_above, cb = sh.sel_cnt;
      __syncthreads();
      prefix |= (uint64_t)bin << shift;
      remaining -= ab;
      if (cb == remaining || shift == 0) break;
    }
    T = prefix;
  }
  __syncthreads();
  // winners: the list above b*, then the bin's keys >= T
  if (threadIdx.x == 0) sh.cnt2 = 0;
  hs_copy(sh.out, a.hwin + row * a.k, nab);
  __syncthreads();
  if (needb > 0 && !spill) {
    for (uint32_t i = threadIdx.x; i < mt.inbin; i += SK_NT) {
      const uint64_t x = sh.cand[i];
      if (x >= T) {
        const uint32_t at = nab + atomicAdd(&sh.cnt2, 1u);
        if (at < (uint32_t)SK_KMAX) sh.out[at] = x;
      }
    }
  } else if (needb > 0) {
    for (int64_t s = threadIdx.x; s < nv; s += SK_NT) {
      const uint64_t x = composite(score_key(src[s]), (uint32_t)s);
      if ((x >> 53) == (pre >> 53) && x >= T) {
        const uint32_t at = nab + atomicAdd(&sh.cnt2, 1u);
        if (at < (uint32_t)SK_KMAX) sh.out[at] = x;
      }
    }
  }
  __syncthreads();
  for (int i = (int)need + threadIdx.x; i < SK_KMAX; i += SK_NT) sh.out[i] = 0;
  __syncthreads();
  bitonic1024_desc(sh.out);
  for (int i = threadIdx.x; i < a.k; i += SK_NT)
    a.idx[grow * a.k + i] = i < (int)need ? (int32_t)(~(uint32_t)sh.out[i]) : -1;
}

// bytes of the histogram-select workspace for `rows` rows of `nparts` parts
static size_t hs_bytes(int64_t rows, int nparts, int k, size_t* o_suf, size_t* o_off, size_t* o_meta,
                       size_t* o_win, size_t* o_cand) {
  auto al = [](size_t x) { return (x + 255) / 256 * 256; };
  size_t o = 0;
  *o_suf = o; o = al(o + (size_t)rows * nparts * HS_BIN * 4);
  *o_off = o; o = al(o + (size_t)rows * nparts * 2 * 4);
  *o_meta = o; o = al(o + (size_t)rows * sizeof(HsMeta));
  *o_win = o; o = al(o + (size_t)rows * k * 8);
  *o_cand = o; o = al(o + (size_t)rows * HS_CAP * 8);
  return o;
}

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

static void topk_plan(int64_t rows, int64_t S, int k, int* part, int* nparts) {
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

size_t topk_workspace_bytes(int64_t rows, int64_t S, int k) {
  int part, nparts;
  if (hs_plan(rows, S, k, &part, &nparts)) {
    size_t o1, o2, o3, o4, o5;
    return hs_bytes(rows, nparts, k, &o1, &o2, &o3, &o4, &o5);
  }
  topk_plan(rows, S, k, &part, &nparts);
  return nparts > 1 ? (size_t)rows * nparts * k * sizeof(uint64_t) : 0;
}

bool topk_supported(int64_t rows, int64_t S, int k) {
  int part, nparts;
  if (k >= 1 && hs_plan(rows, S, k, &part, &nparts)) return true;
  topk_plan(rows, S, k, &part, &nparts);
  return k >= 1 && k <= 4096 && (nparts == 1 || (int64_t)nparts * k <= MAX_CAND);
}

hipError_t launch_topk(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                       const int64_t* q_pos0, int k, int32_t* idx, void* ws, hipStream_t s) {
  if (B <= 0 || nq <= 0) return hipSuccess;
  TopkArgs a = {};
  a.scores = scores; a.nq = nq; a.S = S; a.m = m; a.k = k; a.idx = idx;
  const int64_t rows_l = (B < MAXB ? B : MAXB) * nq;
  if (hs_plan(rows_l, S, k, &a.part, &a.nparts)) {
    size_t o_suf, o_off, o_meta, o_win, o_cand;
    hs_bytes(rows_l, a.nparts, k, &o_suf, &o_off, &o_meta, &o_win, &o_cand);
    uint8_t* w = reinterpret_cast<uint8_t*>(ws);
    a.hsuf = reinterpret_cast<uint32_t*>(w + o_suf);
    a.hoff = reinterpret_cast<uint32_t*>(w + o_off);
    a.hmeta = reinterpret_cast<HsMeta*>(w + o_meta);
    a.hwin = reinterpret_cast<uint64_t*>(w + o_win);
    a.hcand = reinterpret_cast<uint64_t*>(w + o_cand);
    hipError_t e = hipFuncSetAttribute((const void*)topk_h_finish, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(HsShared));
    if (e != hipSuccess) return e;
    for (int64_t b0 = 0; b0 < B; b0 += MAXB) {
      const int nb = (int)(B - b0 < MAXB ? B - b0 : MAXB);
      PosTable pt;
      for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
      const unsigned rows = (unsigned)(nb * nq);
      hipLaunchKernelGGL(topk_h_hist, dim3((unsigned)a.nparts, rows), dim3(SK_NT), 0, s, a, pt, (int)b0);
      hipLaunchKernelGGL(topk_h_thresh, dim3(rows), dim3(SK_NT), 0, s, a, pt, (int)b0);
      hipLaunchKernelGGL(topk_h_compact, dim3((unsigned)a.nparts, rows), dim3(SK_NT), 0, s, a, pt, (int)b0);
      hipLaunchKernelGGL(topk_h_finish, dim3(rows), dim3(SK_NT), sizeof(HsShared), s, a, pt, (int)b0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  topk_plan(rows_l, S, k, &a.part, &a.nparts);
  a.cand = reinterpret_cast<uint64_t*>(ws);
  const int n2 = [&] { int p = 1; while (p < k) p <<= 1; return p; }();
  const bool stream = k <= SK_KMAX;
  const size_t lds1 = stream ? sizeof(SkShared) : (size_t)a.part * 4 + NBIN * 4 + (size_t)n2 * 8;
  const size_t lds2 = (size_t)a.nparts * k * 8 + NBIN * 4 + (size_t)n2 * 8;
  const bool vec = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && S % 4 == 0 && a.part % 4 == 0;
  const void* k1 = !stream ? (const void*)topk_stage1
                           : vec ? (const void*)topk_stream<true> : (const void*)topk_stream<false>;
  hipError_t e = hipFuncSetAttribute(k1, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds1);
  if (e != hipSuccess) return e;
  if (a.nparts > 1) {
    e = hipFuncSetAttribute((const void*)topk_stage2, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds2);
    if (e != hipSuccess) return e;
  }
  for (int64_t b0 = 0; b0 < B; b0 += MAXB) {
    const int nb = (int)(B - b0 < MAXB ? B - b0 : MAXB);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
    if (stream && vec)
      hipLaunchKernelGGL(topk_stream<true>, dim3((unsigned)(nb * nq), (unsigned)a.nparts), dim3(SK_NT), lds1, s,
                         a, pt, (int)b0);
    else if (stream)
      hipLaunchKernelGGL(topk_stream<false>, dim3((unsigned)(nb * nq), (unsigned)a.nparts), dim3(SK_NT), lds1, s,
                         a, pt, (int)b0);
    else
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
