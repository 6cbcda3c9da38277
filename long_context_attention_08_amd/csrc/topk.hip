// Top-k selector (DeepSeek-V4 digest, 模块 B eq 17; jsqmd blog 第二阶段 Top-k稀疏选择).
//
// Every candidate becomes a unique 64-bit composite
//     (order-preserving uint32 key of the fp32 score) << 32  |  ~index
// so "score descending, ties to the lower index" is plain descending order of
// the composite, and the selected set is exactly { x >= T } for the k-th
// largest composite T.  T is found by an MSD radix select in LDS (12-bit
// digits in the k > 1024 stages, 11-bit digits in the streaming and histogram
// selects; each stops as soon as a whole bin is taken), the winners are
// gathered and put in order in LDS: bitonic-sorted by the k > 1024 selects
// and the parts of a split streaming row, ranked by digit bins (rank_by_bins)
// by the streaming select of a whole row, the histogram select and the
// one-call select, which sort only sets with dense ties.
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
#include <mutex>

#include "dsv4_common.h"
#include "dsv4_internal.h"

namespace dsv4 {

// Workspace of the allocation-free top-k call: one array per GPU, zero at
// load and holding the last call's contents afterwards.  Nothing in it needs
// to start at zero: every top-k kernel writes each workspace word before any
// kernel reads it (the counting atomics are in LDS).  Calls that overlap on
// one GPU share it and race.
static __device__ __align__(256) uint8_t scratch[TOPK_SCRATCH_BYTES];

hipError_t topk_scratch_ptr(void** ptr) {
  static std::mutex mu;
  static void* per_dev[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!per_dev[dev]) {
    // the device address of this GPU's copy of the array (its name in host
    // code is only a stand-in)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_dev[dev] = p;
  }
  *ptr = per_dev[dev];
  return hipSuccess;
}

constexpr int TK_THREADS = 1024;
constexpr int NBIN = 4096;

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

struct TopkArgs {
  const float* scores;
  int64_t nq, S;
  int m, k;
  int part;          // scores per stage-1 part
  int nparts;
  int32_t* idx;      // [rows, k]
  uint64_t* cand;    // [rows, nparts, k] (nparts > 1)
  // histogram select (few long rows)
  uint32_t* hsuf;    // [rows, nparts, HS_SUF] suffix counts per part: HS_BIN bins, then every 32nd again
  void* hmeta;       // [rows] HsMeta of the row (threshold bin and counts), 16 bytes each
  uint64_t* hwin;    // [rows, k] winners above the threshold bin
  uint64_t* hcand;   // [rows, HS_CAP] keys of the threshold bin
  const int* flags;  // [rows] or null: rows with a zero flag are skipped
};

// launch-local row `row` is skipped (block-uniform)
__device__ __forceinline__ bool row_skipped(const TopkArgs& a, int64_t row) {
  return a.flags && a.flags[row] == 0;
}

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
  if (row_skipped(a, row)) return;
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
  if (row_skipped(a, row)) return;
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
constexpr int SK_BIN = 2048;                // 11-bit digits

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
constexpr int SK_KSMALL = 512;              // k up to which the streaming select uses the smaller buffer
constexpr int SK_CAP_S = 2560;
static_assert(SK_CAP_S >= SK_STEP + SK_KSMALL && SK_CAP_S % 64 == 0, "the smaller buffer holds a step and k");

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

// the k best of a set of unique composites in order by digit bins (below)
template <int EPT, int CAP>
__device__ bool rank_by_bins(SkSharedT<CAP>& sh, uint32_t* maxc_sh, const uint64_t (&v)[EPT], int n, uint32_t need,
                             int32_t* out);

// dynamic LDS: sizeof(SkSharedT<CAP>).  VEC: every part starts 16-byte
// aligned, so whole steps are read with float4 loads (the last, partial step
// with clamped scalar loads).  CAP candidate slots hold a step next to the k
// kept ones: 3584 for k <= 1024 (37 KB, 4 blocks per CU), 2560 for k <= 512
// (29 KB, 5 blocks per CU; the loop is latency-bound, so more blocks raise the
// rate).  A whole row's k best are put in order by rank_by_bins over the
// buffer (the radix select and bitonic sort only for dense ties).
template <bool VEC, int CAP>
__global__ __launch_bounds__(SK_NT) void topk_stream(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  SkSharedT<CAP>& sh = *reinterpret_cast<SkSharedT<CAP>*>(smem);
  __shared__ uint32_t s_maxc;
  const int64_t row = (int64_t)blockIdx.x;         // row within this launch's batch slice
  if (row_skipped(a, row)) return;
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
    if (sh.cnt > (uint32_t)(CAP - SK_STEP)) compact();
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
  if (a.nparts == 1) {
    constexpr int EPT = (CAP + SK_NT - 1) / SK_NT;
    uint64_t v[EPT];
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      const int i = (int)threadIdx.x + j * SK_NT;
      v[j] = i < n ? sh.cand[i] : 0ull;
    }
    int32_t* dst = a.idx + grow * a.k;
    if (rank_by_bins<EPT>(sh, &s_maxc, v, n, need, dst)) {
      for (int i = (int)need + threadIdx.x; i < a.k; i += SK_NT) dst[i] = -1;
      return;
    }
  }
  if (need > 0) {                     // sh.cand is as it was when rank_by_bins declines
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
// processed in two launches:
//   1. per part: a 2048-bin histogram of the top 11 key bits, stored as suffix
//      counts (keys at or above each bin), every 32nd of them once more in a
//      short coarse array;
//   2. per part: the threshold bin b* (the highest bin whose suffix count over
//      all parts reaches min(k, visible)), found from the coarse counts and
//      then the 32 bins of the coarse step that holds it; the part's write
//      offsets from every part's counts above and in b*; keys above b* go to
//      the winner list, keys in b* to the candidate list, as composites;
//   3. per row: the candidates are cut to the missing count by the exact
//      radix select, and the k winners are put in order.  When b* holds more
//      keys than the candidate list (heavy ties), the select runs over the
//      row in global memory instead.
// The selected set is the same exact set as on every other path.  (Finishing
// a row in the part that completes a count instead of a third launch needs a
// device-scope release per part, whose L2 write-back doubled the decode time.)
constexpr int HS_PER = HS_BIN / SK_NT;     // bins per thread
static_assert(HS_PER == 8 && HS_COARSE * 32 == HS_BIN, "a coarse count every 32 bins, 4 per 32 threads");
constexpr int HS_MAXPARTS = 64;            // parts per row (the plan's bound)

struct HsMeta {
  int bstar;         // threshold bin (-1: every visible score is taken)
  uint32_t above;    // visible keys in bins above bstar (all winners)
  uint32_t inbin;    // visible keys in bin bstar
  uint32_t need;     // min(k, visible)
};
static_assert(sizeof(HsMeta) == 16, "the plan keeps 16 bytes per row");

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
  if (row_skipped(a, row)) return;
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
  uint32_t* dst = a.hsuf + (row * a.nparts + p) * HS_SUF;
#pragma unroll
  for (int q = HS_PER - 1; q >= 0; --q) {
    acc += c[q];
    dst[HS_PER * threadIdx.x + q] = acc;
  }
  if ((threadIdx.x & 3) == 0) dst[HS_BIN + (threadIdx.x >> 2)] = acc;   // bin 32 j = HS_PER * 4 j
}

// global -> LDS copy of n composites, eight loads in flight per thread// global -> LDS copy of n composites, eight loads in flight per thread
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

// Descending order of n unique composites by one pass over digit bins.
// Thread t holds positions t + j SK_NT (j < EPT) of the set in v; positions
// at or past n are ignored.  A histogram of the 11 bits below their highest
// differing bit (so every bin is a contiguous range of composites),
// descending bin offsets, and a scatter that groups each bin into sh.cand;
// then each composite's place is its bin's offset plus the number of larger
// composites in its bin.  Places below `need` are written to out as the
// index (~ low word).  A set where a bin that reaches the first `need`
// places holds more than RANK_BIN_MAX composites (dense ties) returns false
// before the scatter, having written nothing and left sh.cand as it was: the
// caller sorts instead.  sh.hist (and the sh.out it shares memory with) is
// overwritten; maxc is one word (LDS).  One array serves as histogram, bin
// offsets and scatter cursor: the bins are placed from the top, so once the
// scatter has moved each cursor to its bin's end, the start of bin b is the
// cursor of bin b + 1.
constexpr int RANK_BIN_MAX = 64;
template <int EPT, int CAP>
__device__ bool rank_by_bins(SkSharedT<CAP>& sh, uint32_t* maxc_sh, const uint64_t (&v)[EPT], int n, uint32_t need,
                             int32_t* out) {
  uint64_t mn = ~0ull, mx = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    if ((int)threadIdx.x + j * SK_NT < n) {
      mn = v[j] < mn ? v[j] : mn;
      mx = v[j] > mx ? v[j] : mx;
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    const uint64_t p = shfl_xor_u64(mn, o), q = shfl_xor_u64(mx, o);
    mn = p < mn ? p : mn;
    mx = q > mx ? q : mx;
  }
  if ((threadIdx.x & 63) == 0) { sh.rmin[threadIdx.x >> 6] = mn; sh.rmax[threadIdx.x >> 6] = mx; }
  for (int b = threadIdx.x; b < SK_BIN; b += SK_NT) sh.hist[b] = 0;
  if (threadIdx.x == 0) *maxc_sh = 0;
  __syncthreads();
  mn = sh.rmin[0];
  mx = sh.rmax[0];
#pragma unroll
  for (int w = 1; w < SK_NT / 64; ++w) {
    mn = sh.rmin[w] < mn ? sh.rmin[w] : mn;
    mx = sh.rmax[w] > mx ? sh.rmax[w] : mx;
  }
  // bits above the highest differing one are common: an 11-bit digit just
  // below it orders the composites by bins
  const int hb = mn == mx ? 0 : 63 - __clzll(mn ^ mx);
  const int shift = hb >= 10 ? hb - 10 : 0;
  auto digit = [&](uint64_t x) { return (uint32_t)(x >> shift) & (uint32_t)(SK_BIN - 1); };
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((int)threadIdx.x + j * SK_NT < n) atomicAdd(&sh.hist[digit(v[j])], 1u);
  __syncthreads();
  // thread t owns bins [SK_BIN - 8(t+1), SK_BIN - 8t), from the top; its
  // counts become the bins' first places (each thread reads and writes only
  // its own bins here)
  constexpr int PER = SK_BIN / SK_NT;
  uint32_t c[PER];
  uint32_t loc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) { c[q] = sh.hist[SK_BIN - 1 - (PER * threadIdx.x + q)]; loc += c[q]; }
  uint32_t all;
  uint32_t above = sk_scan_excl(loc, sh.wsum, &all);
  uint32_t maxc = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int b = SK_BIN - 1 - (PER * (int)threadIdx.x + q);
    sh.hist[b] = above;                     // the scatter cursor, which ends at the bin's end
    if (above < need && c[q] > maxc) maxc = c[q];
    above += c[q];
  }
  if (maxc > (uint32_t)RANK_BIN_MAX) atomicMax(maxc_sh, maxc);
  __syncthreads();
  if (*maxc_sh != 0) return false;
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if ((int)threadIdx.x + j * SK_NT < n) sh.cand[atomicAdd(&sh.hist[digit(v[j])], 1u)] = v[j];
  __syncthreads();
  // ranks by position in the grouped list: neighbouring threads take
  // neighbouring composites, mostly of one bin, so a bin's reads are
  // broadcasts and a dense bin's work is spread over many threads
  for (int p = threadIdx.x; p < n; p += SK_NT) {
    const uint64_t x = sh.cand[p];
    const uint32_t b = digit(x);
    const uint32_t s = b + 1 < (uint32_t)SK_BIN ? sh.hist[b + 1] : 0u, e = sh.hist[b];
    if (s >= need) continue;
    uint32_t r = 0;
    for (uint32_t q = s; q < e; ++q) r += sh.cand[q] > x ? 1u : 0u;
    if (s + r < need) out[s + r] = (int32_t)(~(uint32_t)x);
  }
  return true;
}

// The last step of a row: the `above` winners listed above the threshold bin
// plus the needed keys of the bin, in order, into the row's indices (block-wide)
__device__ void hs_finish(const TopkArgs& a, int64_t row, int64_t grow, int64_t nv, const HsMeta& mt, HsShared& sh,
                          uint32_t* maxc_sh) {
  uint32_t& s_maxc = *maxc_sh;
  const uint32_t need = mt.need, nab = mt.above;
  const uint32_t needb = need - nab;                 // to take from bin b*
  const bool spill = mt.inbin > (uint32_t)HS_CAP;
  const float* src = a.scores + grow * a.S;
  const uint64_t pre = (uint64_t)(uint32_t)mt.bstar << 53;   // composites of bin b* start with it
  // the winners above b* (nab < k <= SK_KMAX) are loaded now, in flight during the select
  constexpr int WPT = SK_KMAX / SK_NT;
  uint64_t wv[WPT];
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const uint32_t i = threadIdx.x + j * SK_NT;
    wv[j] = i < nab ? a.hwin[row * a.k + i] : 0ull;
  }
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
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const uint32_t i = threadIdx.x + j * SK_NT;
    if (i < nab) sh.out[i] = wv[j];
  }
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
  // the `need` winners in order: ranked by digit bins, or (dense ties) sorted
  constexpr int EPT = SK_KMAX / SK_NT;
  uint64_t v[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = (int)threadIdx.x + j * SK_NT;
    v[j] = i < (int)need ? sh.out[i] : 0ull;
  }
  __syncthreads();                           // sh.out shares memory with sh.hist
  int32_t* dst = a.idx + grow * a.k;
  if (rank_by_bins<EPT>(sh, &s_maxc, v, (int)need, need, dst)) {
    for (int i = (int)need + threadIdx.x; i < a.k; i += SK_NT) dst[i] = -1;
    return;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < EPT; ++j) sh.out[threadIdx.x + j * SK_NT] = v[j];   // zero past `need`
  __syncthreads();
  bitonic1024_desc(sh.out);
  for (int i = threadIdx.x; i < a.k; i += SK_NT) dst[i] = i < (int)need ? (int32_t)(~(uint32_t)sh.out[i]) : -1;
}

__global__ __launch_bounds__(SK_NT) void topk_h_cut(TopkArgs a, PosTable pt, int b0) {
  __shared__ uint32_t s_part[SK_NT];
  __shared__ uint32_t s_tot[HS_COARSE];
  __shared__ uint32_t wsum[SK_NT / 64];
  __shared__ int s_j, s_b;
  __shared__ uint32_t s_offa, s_offb, na, nb;
  const int64_t row = blockIdx.y;
  if (row_skipped(a, row)) return;
  const int p = blockIdx.x;
  const int t = threadIdx.x;
  int64_t nv;
  const int64_t grow = hs_row(a, pt, b0, row, &nv);
  const uint32_t need = (uint32_t)(nv < a.k ? nv : a.k);
  const bool cut = need < (uint64_t)nv;
  const uint32_t* suf = a.hsuf + row * a.nparts * HS_SUF;
  const int64_t s0 = (int64_t)p * a.part, s1 = s0 + a.part < nv ? s0 + a.part : nv;
  const float* src = a.scores + grow * a.S;
  // threshold bin: the highest bin whose suffix count over the parts reaches
  // `need` (suffix counts do not increase with the bin); none when every
  // visible key is taken
  if (t == 0) { s_j = 0; s_b = -1; }
  if (cut) {
    {   // coarse counts: thread g * 64 + j adds count j of parts g, g + 4, ... (all loads in flight)
      const int j = t & (HS_COARSE - 1), g = t / HS_COARSE;
      constexpr int NPC = HS_MAXPARTS / (SK_NT / HS_COARSE);
      uint32_t v[NPC];
#pragma unroll
      for (int i = 0; i < NPC; ++i) {
        const int pp = g + i * (SK_NT / HS_COARSE);
        v[i] = pp < a.nparts ? suf[pp * HS_SUF + HS_BIN + j] : 0u;
      }
      uint32_t sum = 0;
#pragma unroll
      for (int i = 0; i < NPC; ++i) sum += v[i];
      s_part[t] = sum;
    }
    __syncthreads();
    if (t < HS_COARSE) {
      uint32_t tot = 0;
#pragma unroll
      for (int g = 0; g < SK_NT / HS_COARSE; ++g) tot += s_part[g * HS_COARSE + t];
      s_tot[t] = tot;
    }
    __syncthreads();
    if (t < HS_COARSE && s_tot[t] >= need && (t + 1 == HS_COARSE || s_tot[t + 1] < need)) s_j = t;
    __syncthreads();
    const int jc = s_j;
    {   // the 32 bins of coarse step jc: thread g * 32 + i adds bin 32 jc + i of parts g, g + 8, ...
      const int i = t & 31, g = t >> 5;
      constexpr int NPF = HS_MAXPARTS / (SK_NT / 32);
      uint32_t v[NPF];
#pragma unroll
      for (int q = 0; q < NPF; ++q) {
        const int pp = g + q * (SK_NT / 32);
        v[q] = pp < a.nparts ? suf[pp * HS_SUF + 32 * jc + i] : 0u;
      }
      uint32_t sum = 0;
#pragma unroll
      for (int q = 0; q < NPF; ++q) sum += v[q];
      s_part[t] = sum;
    }
    __syncthreads();
    if (t < 32) {
      uint32_t tot = 0;
#pragma unroll
      for (int g = 0; g < SK_NT / 32; ++g) tot += s_part[g * 32 + t];
      s_tot[t] = tot;                      // bins 32 jc .. 32 jc + 31 (coarse counts no longer needed)
    }
    __syncthreads();
    // the bin after 32 jc + 31 is the next coarse step, below need by the choice of jc
    if (t < 32 && s_tot[t] >= need && (t == 31 || s_tot[t + 1] < need)) s_b = 32 * jc + t;
  }
  __syncthreads();
  const int bstar = s_b;
  // every part's keys above and in b*; this part's write offsets
  uint32_t ca = 0, cb = 0;
  if (t < a.nparts) {
    const uint32_t* sp = suf + t * HS_SUF;
    ca = bstar + 1 < HS_BIN ? sp[bstar + 1] : 0u;
    cb = bstar >= 0 ? sp[bstar] - ca : 0u;
  }
  uint32_t ta, tb;
  const uint32_t ea = sk_scan_excl(ca, wsum, &ta);
  const uint32_t eb = sk_scan_excl(cb, wsum, &tb);
  if (t == p) { s_offa = ea; s_offb = eb; }
  if (p == 0 && t == 0) reinterpret_cast<HsMeta*>(a.hmeta)[row] = HsMeta{bstar, ta, tb, need};
  if (t == 0) { na = 0; nb = 0; }
  __syncthreads();
  if (need > 0) {
    const uint32_t offa = s_offa, offb = s_offb;
    uint64_t* win = a.hwin + row * a.k;
    uint64_t* cand = a.hcand + row * HS_CAP;
    auto place = [&](float x, int64_t s) {
      if (s >= s1) return;
      const uint32_t key = score_key(x);
      const int bin = (int)(key >> 21);
      if (bin > bstar) {
        win[offa + atomicAdd(&na, 1u)] = composite(key, (uint32_t)s);
      } else if (bin == bstar) {
        const uint32_t at = offb + atomicAdd(&nb, 1u);
        if (at < (uint32_t)HS_CAP) cand[at] = composite(key, (uint32_t)s);
      }
    };
    for (int64_t base = s0; base < s1; base += 8 * SK_NT) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int64_t s = base + u * SK_NT + t;
        x[u] = src[s < s1 ? s : s1 - 1];
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) place(x[u], base + u * SK_NT + t);
    }
  }
}

// dynamic LDS: sizeof(HsShared)
__global__ __launch_bounds__(SK_NT) void topk_h_finish(TopkArgs a, PosTable pt, int b0) {
  extern __shared__ __align__(16) uint8_t smem[];
  HsShared& sh = *reinterpret_cast<HsShared*>(smem);
  __shared__ uint32_t s_maxc;
  const int64_t row = blockIdx.x;
  if (row_skipped(a, row)) return;
  int64_t nv;
  const int64_t grow = hs_row(a, pt, b0, row, &nv);
  hs_finish(a, row, grow, nv, reinterpret_cast<const HsMeta*>(a.hmeta)[row], sh, &s_maxc);
}

hipError_t launch_topk(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                       const int64_t* q_pos0, int k, int32_t* idx, void* ws, const TopkPlan& plan, hipStream_t s) {
  return launch_topk_rows(scores, B, nq, S, m, q_pos0, k, idx, ws, plan, nullptr, s);
}

hipError_t launch_topk_rows(const float* scores, int64_t B, int64_t nq, int64_t S, int m,
                            const int64_t* q_pos0, int k, int32_t* idx, void* ws, const TopkPlan& plan,
                            const int* row_flags, hipStream_t s) {
  if (B <= 0 || nq <= 0) return hipSuccess;
  if (row_flags && B > MAXB) return hipErrorInvalidValue;     // flags index the rows of one launch slice
  TopkArgs a = {};
  a.scores = scores; a.nq = nq; a.S = S; a.m = m; a.k = k; a.idx = idx;
  a.flags = row_flags;
  a.part = plan.part;
  a.nparts = plan.nparts;
  if (plan.kind == TOPK_HIST) {
    if (plan.nparts > HS_MAXPARTS || plan.nparts > SK_NT) return hipErrorInvalidValue;   // the cut pass's bound
    uint8_t* w = reinterpret_cast<uint8_t*>(ws);
    a.hsuf = reinterpret_cast<uint32_t*>(w + plan.o_suf);
    a.hmeta = w + plan.o_meta;
    a.hwin = reinterpret_cast<uint64_t*>(w + plan.o_win);
    a.hcand = reinterpret_cast<uint64_t*>(w + plan.o_cand);
    hipError_t e = hipFuncSetAttribute((const void*)topk_h_finish, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       (int)sizeof(HsShared));
    if (e != hipSuccess) return e;
    for (int64_t b0 = 0; b0 < B; b0 += MAXB) {
      const int nb = (int)(B - b0 < MAXB ? B - b0 : MAXB);
      PosTable pt;
      for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = q_pos0[b0 + i]; pt.win_pos0[i] = 0; }
      const unsigned rows = (unsigned)(nb * nq);
      hipLaunchKernelGGL(topk_h_hist, dim3((unsigned)a.nparts, rows), dim3(SK_NT), 0, s, a, pt, (int)b0);
      hipLaunchKernelGGL(topk_h_cut, dim3((unsigned)a.nparts, rows), dim3(SK_NT), 0, s, a, pt, (int)b0);
      hipLaunchKernelGGL(topk_h_finish, dim3(rows), dim3(SK_NT), sizeof(HsShared), s, a, pt, (int)b0);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    return hipSuccess;
  }
  a.cand = reinterpret_cast<uint64_t*>(ws);
  const int n2 = [&] { int p = 1; while (p < k) p <<= 1; return p; }();
  const bool stream = plan.kind == TOPK_STREAM;
  const bool small = k <= SK_KSMALL;     // the smaller candidate buffer
  const size_t lds1 = stream ? (small ? sizeof(SkSharedT<SK_CAP_S>) : sizeof(SkShared))
                             : (size_t)a.part * 4 + NBIN * 4 + (size_t)n2 * 8;
  const size_t lds2 = (size_t)a.nparts * k * 8 + NBIN * 4 + (size_t)n2 * 8;
  const bool vec = (reinterpret_cast<uintptr_t>(scores) & 15) == 0 && S % 4 == 0 && a.part % 4 == 0;
  const void* k1 = !stream ? (const void*)topk_stage1
                   : vec   ? (small ? (const void*)topk_stream<true, SK_CAP_S> : (const void*)topk_stream<true, SK_CAP>)
                           : (small ? (const void*)topk_stream<false, SK_CAP_S> : (const void*)topk_stream<false, SK_CAP>);
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
    const dim3 g1((unsigned)(nb * nq), (unsigned)a.nparts);
    if (stream && vec && small)
      hipLaunchKernelGGL((topk_stream<true, SK_CAP_S>), g1, dim3(SK_NT), lds1, s, a, pt, (int)b0);
    else if (stream && vec)
      hipLaunchKernelGGL((topk_stream<true, SK_CAP>), g1, dim3(SK_NT), lds1, s, a, pt, (int)b0);
    else if (stream && small)
      hipLaunchKernelGGL((topk_stream<false, SK_CAP_S>), g1, dim3(SK_NT), lds1, s, a, pt, (int)b0);
    else if (stream)
      hipLaunchKernelGGL((topk_stream<false, SK_CAP>), g1, dim3(SK_NT), lds1, s, a, pt, (int)b0);
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

// ------------------------------------------------------------------ index scores and top-k in one call

// the float whose order key is `key` (finite or -inf for every key a
// finite score or a prefix of one can have)
__device__ __forceinline__ float key_to_float(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Row thresholds from the sample top-k (long sample rows): the ks-th best
// sample score, or -inf (every visible score passes) when the row sees fewer
// than ks sample keys
__global__ void it_lkey(const float* sscore, const int32_t* sidx, int64_t rows, int64_t Ss, int ks, float* lval) {
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= rows) return;
  const int32_t j = sidx[r * ks + ks - 1];
  lval[r] = j >= 0 ? key_to_float(score_key(sscore[r * Ss + j])) : -INFINITY;
}

constexpr int IT_THRESH_MAX = 16384;   // sample scores a threshold block holds in LDS

// Row thresholds straight from the sample scores (rows of at most
// IT_THRESH_MAX): one block per row stages the visible sample keys in LDS and
// runs an MSD radix select (11, 11, 10 bits) for the ks-th largest key.  It
// stops early when a whole digit bin is taken; the threshold is then the bin's
// lowest key, with exactly ks sample keys at or above it.  Either way at
// least ks sample scores reach the threshold.  dynamic LDS: Ss * 4 bytes
__global__ __launch_bounds__(SK_NT) void it_thresh(const float* sscore, int64_t nq, int64_t Ss, int m, int ks,
                                                    PosTable pt, float* lval) {
  extern __shared__ __align__(16) uint32_t keys[];
  __shared__ uint32_t hist[SK_BIN];
  __shared__ uint32_t wsum[SK_NT / 64];
  __shared__ uint32_t sel_bin, sel_above, sel_cnt;
  const int64_t row = blockIdx.x;
  const int64_t bl = row / nq, t = row % nq;
  const int nv = (int)visible_count(pt.q_pos0[bl] + t, m, Ss);
  if (nv < ks) {
    if (threadIdx.x == 0) lval[row] = -INFINITY;
    return;
  }
  const float* src = sscore + row * Ss;
  for (int base = 0; base < nv; base += 8 * SK_NT) {      // eight loads in flight per thread
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * SK_NT + (int)threadIdx.x;
      x[u] = src[i < nv ? i : nv - 1];
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = base + u * SK_NT + (int)threadIdx.x;
      if (i < nv) keys[i] = score_key(x[u]);
    }
  }
  uint32_t prefix = 0, remaining = (uint32_t)ks;
  int shift = 32;
  for (int level = 0; level < 3; ++level) {
    const int width = level < 2 ? 11 : 10;
    shift -= width;
    const int top = shift + width;
    for (int i = threadIdx.x; i < SK_BIN; i += SK_NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < nv; i += SK_NT) {
      const uint32_t k = keys[i];
      if (top >= 32 || (k >> top) == (prefix >> top)) atomicAdd(&hist[(k >> shift) & ((1u << width) - 1u)], 1u);
    }
    __syncthreads();
    constexpr int PER = SK_BIN / SK_NT;
    uint32_t c[PER];
    uint32_t loc = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) { c[q] = hist[SK_BIN - 1 - (PER * threadIdx.x + q)]; loc += c[q]; }
    uint32_t total;
    uint32_t above = sk_scan_excl(loc, wsum, &total);
    if (above < remaining && remaining <= above + loc) {
#pragma unroll
      for (int q = 0; q < PER; ++q) {
        if (above < remaining && remaining <= above + c[q]) {
          sel_bin = SK_BIN - 1 - (PER * threadIdx.x + q);
          sel_above = above;
          sel_cnt = c[q];
        }
        above += c[q];
      }
    }
    __syncthreads();
    const uint32_t bin = sel_bin, ab = sel_above, cb = sel_cnt;
    __syncthreads();
    prefix |= bin << shift;
    remaining -= ab;
    if (cb == remaining) break;          // the whole bin is taken
  }
  if (threadIdx.x == 0) lval[row] = key_to_float(prefix);
}

struct ItSelArgs {
  const uint64_t* cand;     // [rows, splits, cap] composites
  const uint32_t* ccount;   // [rows, splits] list lengths (may exceed cap)
  int splits, cap;
  int64_t nq, S;
  int m, k;
  int32_t* idx;             // [rows, k]
  int* flags;               // [rows] out: 1 = left to the full-score path
};

static_assert(IT_SELCAP == SK_CAP, "a select block holds the candidates of one row");
// the smaller select block, taken where the expected candidates of a row
// (IT_STRIDE ks) leave it the margin (8/5) the one-call path asks of the larger
constexpr int IT_CAP_S = 2944;
static_assert(IT_CAP_S <= SK_CAP && IT_CAP_S % 64 == 0, "the smaller select block");
static bool it_small_select(int ks) { return (int64_t)IT_STRIDE * ks * 8 / 5 <= IT_CAP_S; }

// One block per row: the k best of the row's lists, sorted.  Every visible
// score at or above the row's threshold is in the lists unless one
// overflowed; when there are at least min(k, visible) of them, the k best
// of the row are among them.  A row where either fails, or whose lists
// exceed one block's buffer, is flagged and left to the full-score path.
//
// The lists' composites are ranked in one pass by digit bins (rank_by_bins);
// a row with dense ties there takes the radix select and the bitonic sort
// instead; both give the same sorted list.
//
// CAP composites fit the block's LDS: 3584 (37 KB, 4 blocks per CU), or,
// where the expected candidates are fewer, IT_CAP_S (32 KB, 5 blocks per CU:
// the block is a latency chain, so the rate follows the blocks per CU).  The
// list counts and offsets of the loading phase live in sh.hist, which the
// ranking only uses afterwards.
template <int CAP>
__global__ __launch_bounds__(SK_NT) void it_select(ItSelArgs a, PosTable pt) {
  constexpr int EPT = (CAP + SK_NT - 1) / SK_NT;   // composites per thread
  extern __shared__ __align__(16) uint8_t smem[];
  SkSharedT<CAP>& sh = *reinterpret_cast<SkSharedT<CAP>*>(smem);
  static_assert(2 * SK_NT <= SK_BIN, "list counts and offsets fit the histogram's space");
  uint32_t* const s_cnt = sh.hist;
  uint32_t* const s_off = sh.hist + SK_NT;
  __shared__ uint32_t s_maxc;
  const int64_t row = blockIdx.x;
  const int64_t bl = row / a.nq, t = row % a.nq;
  const int64_t nv = visible_count(pt.q_pos0[bl] + t, a.m, a.S);
  const uint32_t need = (uint32_t)(nv < a.k ? nv : a.k);
  const uint32_t* cnt = a.ccount + row * a.splits;
  uint32_t tot = 0;
  int over = 0;
  for (int i = threadIdx.x; i < a.splits; i += SK_NT) {
    const uint32_t c = cnt[i];
    tot += c;
    over |= c > (uint32_t)a.cap ? 1 : 0;
  }
  uint32_t total;
  sk_scan_excl(tot, sh.wsum, &total);
  const bool flag = __syncthreads_or(over) || total < need || total > (uint32_t)CAP;
  if (threadIdx.x == 0) a.flags[row] = flag ? 1 : 0;
  if (flag) return;
  int32_t* out = a.idx + row * a.k;
  if (need == 0) {
    for (int i = threadIdx.x; i < a.k; i += SK_NT) out[i] = -1;
    return;
  }
  // the lists into LDS, SK_NT lists at a time: offsets from a block scan of
  // their lengths, then one wave copies each list
  uint32_t base = 0;
  for (int c0 = 0; c0 < a.splits; c0 += SK_NT) {
    const int i = c0 + (int)threadIdx.x;
    const uint32_t c = i < a.splits ? cnt[i] : 0u;
    uint32_t sum;
    const uint32_t ex = sk_scan_excl(c, sh.wsum, &sum);
    s_cnt[threadIdx.x] = c;
    s_off[threadIdx.x] = base + ex;
    __syncthreads();
    const int nsp = a.splits - c0 < SK_NT ? a.splits - c0 : SK_NT;
    // flat positions [base, base + sum): list j holds [s_off[j], s_off[j] + s_cnt[j]);
    // eight loads in flight per thread
    const uint64_t* lists = a.cand + ((uint64_t)row * a.splits + c0) * (uint64_t)a.cap;
    for (uint32_t p0 = base; p0 < base + sum; p0 += 8 * SK_NT) {
      uint64_t v[8];
      uint32_t at[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = p0 + u * SK_NT + threadIdx.x;
        at[u] = p;
        int lo = 0, hi = nsp - 1;                  // last list starting at or before p
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (s_off[mid] <= p) lo = mid;
          else hi = mid - 1;
        }
        v[u] = p < base + sum ? lists[(uint64_t)lo * a.cap + (p - s_off[lo])] : 0ull;
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (at[u] < base + sum) sh.cand[at[u]] = v[u];
    }
    __syncthreads();
    base += sum;
  }
  const int n = (int)total;
  // ---- one-pass rank by digit bins
  uint64_t v[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int i = (int)threadIdx.x + j * SK_NT;
    v[j] = i < n ? sh.cand[i] : 0ull;
  }
  if (rank_by_bins<EPT>(sh, &s_maxc, v, n, need, out)) {
    for (int i = (int)need + threadIdx.x; i < a.k; i += SK_NT) out[i] = -1;
    return;
  }
  // ---- dense ties: radix select, gather, bitonic sort (sh.cand is untouched)
  const uint64_t T = sk_select(sh, n, need);
  sk_gather(sh, n, T);
  const int n2 = pow2_ceil(a.k) > 256 ? SK_KMAX : pow2_ceil(a.k);
  for (int i = need + threadIdx.x; i < n2; i += SK_NT) sh.out[i] = 0;
  __syncthreads();
  if (n2 == SK_KMAX) bitonic1024_desc(sh.out);
  else bitonic_desc<SK_NT>(sh.out, n2);
  for (int i = threadIdx.x; i < a.k; i += SK_NT) out[i] = i < (int)need ? (int32_t)(~(uint32_t)sh.out[i]) : -1;
}

hipError_t launch_indexer_topk(const IndexerArgs& a0, const int64_t* q_pos0, int k, int32_t* idx, void* ws,
                               hipStream_t s) {
  if (a0.B <= 0 || a0.nq <= 0) return hipSuccess;
  const size_t qes = a0.q_dtype == ACT_F32 ? 4 : 2;
  const bool mx = a0.k_layout == ROW_MXFP4;
  const size_t krow = mx ? (size_t)a0.cI / 2 : (size_t)row_bytes(a0.k_layout, a0.cI);
  uint8_t* w = reinterpret_cast<uint8_t*>(ws);
  hipError_t e = hipFuncSetAttribute((const void*)it_select<SK_CAP>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)sizeof(SkShared));
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)it_select<IT_CAP_S>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)sizeof(SkSharedT<IT_CAP_S>));
  if (e != hipSuccess) return e;
#define IT_CHECK(x)            \
  do {                         \
    hipError_t e_ = (x);       \
    if (e_ != hipSuccess) return e_; \
  } while (0)
  for (int64_t b0 = 0; b0 < a0.B; b0 += MAXB) {
    const int nb = (int)(a0.B - b0 < MAXB ? a0.B - b0 : MAXB);
    IndexerArgs a = a0;
    a.qI = reinterpret_cast<const uint8_t*>(a0.qI) + (size_t)b0 * a0.nq * a0.hI * a0.cI * qes;
    a.wI = a0.wI + b0 * a0.nq * a0.hI;
    a.keys = reinterpret_cast<const uint8_t*>(a0.keys) + (size_t)b0 * a0.S * krow;
    a.k_scales = mx ? a0.k_scales + (size_t)b0 * a0.S * (a0.cI / 32) : nullptr;
    a.B = nb;
    a.scores = nullptr;
    a.cand = nullptr; a.ccount = nullptr; a.lval = nullptr; a.cap = 0; a.row_flags = nullptr;
    const int64_t* qp = q_pos0 + b0;
    int32_t* oidx = idx + b0 * a0.nq * k;
    const int64_t rows = (int64_t)nb * a.nq;
    const IdxTopkPlan p = idxtopk_make_plan(a, k);
    float* scores = reinterpret_cast<float*>(w + p.o_scores);
    if (!p.fused) {
      IndexerArgs af = a;
      af.scores = scores;
      IT_CHECK(launch_indexer(af, qp, s));
      IT_CHECK(launch_topk(scores, nb, a.nq, a.S, a.m, qp, k, oidx, w + p.o_ftk, p.tk_full, s));
      continue;
    }
    // sample scores (keys 32 j + 31, read in place) and their ks-th best per row
    IndexerArgs as = a;
    as.S = p.Ss;
    as.kbatch = a.S;
    as.koff = IT_STRIDE - 1;
    as.kstride = IT_STRIDE;
    as.m = a.m * IT_STRIDE;
    as.scores = reinterpret_cast<float*>(w + p.o_sscore);
    IT_CHECK(launch_indexer(as, qp, s));
    float* lval = reinterpret_cast<float*>(w + p.o_lkey);
    PosTable pt;
    for (int i = 0; i < nb; ++i) { pt.q_pos0[i] = qp[i]; pt.win_pos0[i] = 0; }
    if (p.Ss <= IT_THRESH_MAX) {
      const size_t lds = (size_t)p.Ss * 4;
      IT_CHECK(hipFuncSetAttribute((const void*)it_thresh, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
      hipLaunchKernelGGL(it_thresh, dim3((unsigned)rows), dim3(SK_NT), lds, s, as.scores, a.nq, p.Ss, as.m, p.ks, pt,
                         lval);
    } else {
      int32_t* sidx = reinterpret_cast<int32_t*>(w + p.o_sidx);
      IT_CHECK(launch_topk(as.scores, nb, a.nq, p.Ss, as.m, qp, p.ks, sidx, w + p.o_stk, p.tk_sample, s));
      hipLaunchKernelGGL(it_lkey, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, as.scores, sidx, rows,
                         p.Ss, p.ks, lval);
    }
    IT_CHECK(hipGetLastError());
    // full pass: candidate lists
    IndexerArgs ae = a;
    ae.cand = reinterpret_cast<uint64_t*>(w + p.o_cand);
    ae.ccount = reinterpret_cast<uint32_t*>(w + p.o_cnt);
    ae.lval = lval;
    ae.cap = p.cap;
    IT_CHECK(launch_indexer(ae, qp, s));
    // per-row select; flagged rows take the full-score path
    int* flags = reinterpret_cast<int*>(w + p.o_flags);
    ItSelArgs sa{ae.cand, ae.ccount, p.grid.splits, p.cap, a.nq, a.S, a.m, k, oidx, flags};
    if (it_small_select(p.ks))
      hipLaunchKernelGGL((it_select<IT_CAP_S>), dim3((unsigned)rows), dim3(SK_NT), sizeof(SkSharedT<IT_CAP_S>), s,
                         sa, pt);
    else
      hipLaunchKernelGGL((it_select<SK_CAP>), dim3((unsigned)rows), dim3(SK_NT), sizeof(SkShared), s, sa, pt);
    IT_CHECK(hipGetLastError());
    IndexerArgs af = a;
    af.scores = scores;
    af.row_flags = flags;
    IT_CHECK(launch_indexer(af, qp, s));
    IT_CHECK(launch_topk_rows(scores, nb, a.nq, a.S, a.m, qp, k, oidx, w + p.o_ftk, p.tk_full, flags, s));
  }
#undef IT_CHECK
  return hipSuccess;
}

}  // namespace dsv4
